// quantize.hip -- key write and query preparation for the lightning indexer (gfx950).
//
// Implements rotate_activation + act_quant of Indexer.forward (page "Hadamard
// rotation": kbar = ktilde (1/sqrt 128) H_128, bf16 in and out, then fp8
// quantization in groups of 128 features; page "Index key cache": e4m3fn values
// with one float32 power-of-two scale per 128 features) and, for queries, the
// weight fold of page "Index scores" (1/sqrt(128) folded with each query's scale).
//
// Layout: 8 lanes own one 128-feature row, 16 features per lane (feature
// i = 16 * lane_in_row + e), so a wave handles 8 rows and every global access is a
// contiguous 16-byte vector.  The Walsh-Hadamard butterflies run in fp64: the
// inputs have 8-bit significands, so every partial sum is exact whenever the row's
// magnitudes span at most 2^38, and the result does not depend on butterfly order.
// Bits 0-3 of the feature index are combined in registers, bits 4-6 across the 8
// lanes with xor-shuffles.
#include "lk_device.h"

#pragma clang fp contract(off)

namespace lk {
namespace {

constexpr int kRowsPerBlock = 32;  // 256 threads, 8 lanes per row
constexpr double kRotScale = 0x1.6a09e667f3bcdp-4;  // fl64(128 ** -0.5)
constexpr float kSoftmaxScale = 0x1.6a09e6p-4f;     // fl32(128 ** -0.5)

__device__ __forceinline__ double bf16_bits_to_double(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

// Round to the nearest bf16 value, ties to even, straight from fp64.
__device__ __forceinline__ double round_to_bf16(double p) {
    int e = __builtin_amdgcn_frexp_exp(p) - 1;  // 2^e <= |p| < 2^(e+1); p == 0 gives -1
    e = e < -126 ? -126 : e;                    // bf16 subnormal spacing is 2^-133
    return __builtin_ldexp(__builtin_rint(__builtin_ldexp(p, 7 - e)), e - 7);
}

// e4m3fn code of q, |q| <= 448: nearest-even, sign kept, never NaN.
__device__ __forceinline__ uint32_t encode_e4m3(float q) {
    float a = __builtin_fabsf(q);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);  // subnormals: multiples of 2^-9 (8 -> 0x08 = 2^-6)
    } else {
        int e = __builtin_amdgcn_frexp_expf(a) - 1;    // 2^e <= a < 2^(e+1), -6 <= e <= 8
        uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
        code = (uint32_t)((e + 7) << 3) + m - 8;       // m == 16 carries into the exponent
    }
    return code | (__float_as_uint(q) >> 24 & 0x80u);
}

// Quantize the row owned by this 8-lane group.  `in` holds the lane's 16 bf16 bit
// patterns (8 dwords).  Returns the 16 codes packed in 4 dwords and the exponent j.
__device__ __forceinline__ void quantize_row16(const uint32_t in[8], uint32_t out[4], int &j_out) {
    double x[16];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        x[2 * i] = bf16_bits_to_double(in[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_bits_to_double(in[i] >> 16);
    }
    // In-lane butterflies: feature-index bits 0..3.
#pragma unroll
    for (int b = 1; b < 16; b <<= 1) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            if (e & b) continue;
            double u = x[e], v = x[e | b];
            x[e] = u + v;
            x[e | b] = u - v;
        }
    }
    // Cross-lane butterflies: feature-index bits 4..6 = lane bits 0..2.
    const int lane = __lane_id();
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 16; e++) {
            double y = __shfl_xor(x[e], m, 64);
            x[e] = upper ? (y - x[e]) : (x[e] + y);
        }
    }
    // Scale, round to bf16, amax.
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
        double r = x[e] == 0.0 ? 0.0 : x[e];   // an exact zero sum is +0
        double y = round_to_bf16(r * kRotScale);
        x[e] = y;
        amax = __builtin_fmax(amax, __builtin_fabs(y));
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) amax = __builtin_fmax(amax, __shfl_xor(amax, m, 64));
    // Smallest j >= -126 with amax <= 448 * 2^j.  amax = f * 2^E with f in [0.5, 1):
    // j = E - 9 if f <= 0.875 (448 = 0.875 * 2^9), else E - 8.
    int j = -126;
    if (amax > 0.0) {
        int E = __builtin_amdgcn_frexp_exp(amax);
        double f = __builtin_amdgcn_frexp_mant(amax);
        j = E - 9 + (f > 0.875 ? 1 : 0);
        j = j < -126 ? -126 : j;
    }
    j_out = j;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            float q = (float)__builtin_ldexp(x[4 * i + k], -j);  // exact for every value that can encode nonzero
            w |= encode_e4m3(q) << (8 * k);
        }
        out[i] = w;
    }
}

struct KeyJob {
    const uint16_t *x;
    int64_t n_seq, n_rows, x_seq_stride;
    uint8_t *cache;
    float *cache_scale;
    int64_t cache_seq_stride, cache_rows, row_offset;
    const int32_t *positions;
};

struct QueryJob {
    const uint16_t *q;
    const float *w;
    int64_t n_rows;
    uint8_t *q_fp8;
    float *w_eff, *q_scale;
};

// Row g of the key job, owned by the 8 lanes of this row group (sub = lane in group).
__device__ __forceinline__ void key_row(const KeyJob &k, int64_t g, int sub) {
    const int64_t b = g / k.n_rows;
    const int64_t i = g - b * k.n_rows;
    const uint4 *src = reinterpret_cast<const uint4 *>(k.x + (b * k.x_seq_stride + i) * LK_DIM + sub * 16);
    uint4 v0 = src[0], v1 = src[1];
    uint32_t in[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t out[4];
    int j;
    quantize_row16(in, out, j);
    const int64_t p = (k.positions ? (int64_t)k.positions[b] : k.row_offset) + i;
    if (p < 0 || p >= k.cache_rows) return;
    const int64_t row = b * k.cache_seq_stride + p;
    *reinterpret_cast<uint4 *>(k.cache + row * LK_DIM + sub * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    if (sub == 0) k.cache_scale[row] = __builtin_ldexpf(1.0f, j);
}

__device__ __forceinline__ void query_row(const QueryJob &q, int64_t g, int sub) {
    const uint4 *src = reinterpret_cast<const uint4 *>(q.q + g * LK_DIM + sub * 16);
    uint4 v0 = src[0], v1 = src[1];
    uint32_t in[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t out[4];
    int j;
    quantize_row16(in, out, j);
    *reinterpret_cast<uint4 *>(q.q_fp8 + g * LK_DIM + sub * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    if (sub == 0) {
        const float s = __builtin_ldexpf(1.0f, j);
        const float ws = __fmul_rn(q.w[g], s);        // exact unless it leaves the float range
        q.w_eff[g] = __fmul_rn(ws, kSoftmaxScale);
        if (q.q_scale) q.q_scale[g] = s;
    }
}

// Blocks [0, key_blocks) write keys, the rest quantize queries.  A row group past its
// job's end does no work (no shuffle crosses row groups, so a group is either fully
// valid or fully idle).
__global__ void __launch_bounds__(256)
quantize_kernel(KeyJob kj, QueryJob qj, int64_t key_blocks) {
    const int sub = threadIdx.x & 7;
    if ((int64_t)blockIdx.x < key_blocks) {
        const int64_t g = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 3);
        if (g < kj.n_seq * kj.n_rows) key_row(kj, g, sub);
    } else {
        const int64_t g = ((int64_t)blockIdx.x - key_blocks) * kRowsPerBlock + (threadIdx.x >> 3);
        if (g < qj.n_rows) query_row(qj, g, sub);
    }
}

}  // namespace

// Either job may be empty (n rows == 0); one launch covers both.
hipError_t launch_quantize(const KeyJobArgs &ka, const QueryJobArgs &qa, hipStream_t stream) {
    KeyJob kj{ka.x, ka.n_seq, ka.n_rows, ka.x_seq_stride, ka.cache, ka.cache_scale, ka.cache_seq_stride,
              ka.cache_rows, ka.row_offset, ka.positions};
    QueryJob qj{qa.q, qa.w, qa.n_rows, qa.q_fp8, qa.w_eff, qa.q_scale};
    const int64_t key_blocks = (ka.n_seq * ka.n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t query_blocks = (qa.n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    return launch(quantize_kernel, dim3((unsigned)(key_blocks + query_blocks)), dim3(256), 0u, stream, kj, qj,
                  key_blocks);
}

}  // namespace lk

// quantize.hip -- key write and query preparation for the lightning indexer (gfx950).
//
// Implements rotate_activation + act_quant of Indexer.forward (page "Hadamard
// rotation": kbar = ktilde (1/sqrt 128) H_128, bf16 in and out, then fp8
// quantization in groups of 128 features; page "Index key cache": e4m3fn values
// with one float32 power-of-two scale per 128 features) and, for queries, the
// weight fold of page "Index scores" (1/sqrt(128) folded with each query's scale).
//
// The per-row arithmetic (rotation, bf16 rounding, e4m3fn codes, power-of-two
// scale) lives in quant_device.h; here 8 lanes own one row, 32 rows per block.
#include "lk_device.h"
#include "quant_device.h"

#pragma clang fp contract(off)

namespace lk {
namespace {

constexpr int kRowsPerBlock = 32;  // 256 threads, 8 lanes per row

struct KeyJob {
    const uint16_t *x;
    int64_t n_seq, n_rows, x_seq_stride;
    uint8_t *cache;
    float *cache_scale;
    int64_t cache_seq_stride, cache_rows, row_offset;
    const int32_t *positions;
    const float *rope_cos, *rope_sin;
};

struct QueryJob {
    const uint16_t *q;
    const float *w;
    int64_t n_rows;
    uint8_t *q_fp8;
    float *w_eff, *q_scale;
    int64_t heads;
    const float *rope_cos, *rope_sin;
};

// Row g of the key job, owned by the 8 lanes of this row group (sub = lane in group).
__device__ __forceinline__ void key_row(const KeyJob &k, int64_t g, int sub) {
    const int64_t b = g / k.n_rows;
    const int64_t i = g - b * k.n_rows;
    const uint4 *src = reinterpret_cast<const uint4 *>(k.x + (b * k.x_seq_stride + i) * LK_DIM + sub * 16);
    uint4 v0 = src[0], v1 = src[1];
    const int64_t p = (k.positions ? (int64_t)k.positions[b] : k.row_offset) + i;   // loaded with the row
    uint32_t in[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (k.rope_cos) {
        Rope16 r;
        load_rope16(k.rope_cos + g * (LK_ROPE_DIM / 2), k.rope_sin + g * (LK_ROPE_DIM / 2), sub, r);
        rope_row16(in, r, sub);
    }
    uint32_t out[4];
    int j;
    quantize_row16<2>(in, out, j);
    if (p < 0 || p >= k.cache_rows) return;
    const int64_t row = b * k.cache_seq_stride + p;
    *reinterpret_cast<uint4 *>(k.cache + row * LK_DIM + sub * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    if (sub == 0) k.cache_scale[row] = __builtin_ldexpf(1.0f, j);
}

__device__ __forceinline__ void query_row(const QueryJob &q, int64_t g, int sub) {
    const uint4 *src = reinterpret_cast<const uint4 *>(q.q + g * LK_DIM + sub * 16);
    uint4 v0 = src[0], v1 = src[1];
    const float wg = q.w[g];                           // with the row's loads, not after the rotation
    uint32_t in[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (q.rope_cos) {
        const int64_t tok = g / q.heads;
        Rope16 r;
        load_rope16(q.rope_cos + tok * (LK_ROPE_DIM / 2), q.rope_sin + tok * (LK_ROPE_DIM / 2), sub, r);
        rope_row16(in, r, sub);
    }
    uint32_t out[4];
    int j;
    quantize_row16<2>(in, out, j);
    *reinterpret_cast<uint4 *>(q.q_fp8 + g * LK_DIM + sub * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    if (sub == 0) {
        q.w_eff[g] = fold_weight(wg, j);
        if (q.q_scale) q.q_scale[g] = __builtin_ldexpf(1.0f, j);
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
              ka.cache_rows, ka.row_offset, ka.positions, ka.rope_cos, ka.rope_sin};
    QueryJob qj{qa.q, qa.w, qa.n_rows, qa.q_fp8, qa.w_eff, qa.q_scale, qa.heads > 0 ? qa.heads : 1,
                qa.rope_cos, qa.rope_sin};
    const int64_t key_blocks = (ka.n_seq * ka.n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t query_blocks = (qa.n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    return launch(quantize_kernel, dim3((unsigned)(key_blocks + query_blocks)), dim3(256), 0u, stream, kj, qj,
                  key_blocks);
}

}  // namespace lk

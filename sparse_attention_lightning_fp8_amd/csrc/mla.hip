// mla.hip -- sparse MLA decode attention over the indexer's selected keys (gfx950).
//
// Page "Join query parts" (the MQA-decode excerpt): for one decode token of sequence
// b and head h, logits s_t = scale * (qc_h . c_t + qr_h . r_t) over the cached latent
// rows c_t (512 features) and rotary rows r_t (64 features), the index mask leaves
// only the top-k selected slots t in I, p = softmax(s) over I, o_h = sum_t p_t c_t
// (512 features; the up-projection that follows is outside this path).
//
// Split kernel: block (split, head half, b) owns 64 heads (4 waves x 16) and one
// split of at most 256 entries of the row's index list, taken as chunks of 32 keys.
// A chunk's latent and rotary rows are gathered from HBM into LDS twice: key-major
// (the B operand of S = Q K^T, 8 consecutive features per lane) and feature-major
// (the B operand of O += P V, 8 consecutive keys per lane), the second through an
// 8 x 8 transpose in registers.  Each wave keeps its 16 heads' query (576 features,
// bf16) in registers as the A operand of v_mfma_f32_16x16x32_bf16, runs an online
// softmax over its heads (row max and sum over the 16 lanes that hold one head's
// keys), rounds p to bf16 for the P V product, and accumulates o for 16 heads x 512
// features (128 accumulators per lane).  The split writes its unnormalised o with the
// running max m and sum l to the workspace.
// Combine kernel: per (b, h), o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
#include "lk_device.h"

namespace lk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kH = LK_MLA_HEADS;          // 128
constexpr int kDc = LK_MLA_LATENT;        // 512
constexpr int kDr = LK_MLA_ROPE;          // 64
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerBlock = 16 * kWaves;   // 64
constexpr int kChunk = 32;                    // keys per LDS chunk
constexpr int kSplit = 256;                   // index-list entries per block
constexpr int kLatPitch = 2 * kDc + 16;       // key-major latent row (bytes)
constexpr int kRopePitch = 2 * kDr + 16;      // key-major rotary row (bytes)
constexpr int kTPitch = 2 * kChunk;           // feature-major row: 32 keys (bytes)
static_assert(kThreads == (kChunk / 8) * (kDc / 8), "one 8x8 tile of the chunk per thread");

struct MlaArgs {
    const uint16_t *q_lat, *q_rope;           // [B][128][512], [B][128][64]
    const uint16_t *kv_lat, *kv_rope;         // [B][stride][512], [B][stride][64]
    int64_t stride, cap;
    const int32_t *idx;                       // [B][n_idx]
    int32_t n_idx, nsplit;
    float scale;
    float *o_part;                            // [B][nsplit][128][512]
    float *ml_part;                           // [B][nsplit][128][2]
    float *out;                               // [B][128][512]
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t dword_of(const uint4 &v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// Max / sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), result in every lane.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 1, 64));
    x = fmaxf(x, __shfl_xor(x, 2, 64));
    x = fmaxf(x, __shfl_xor(x, 4, 64));
    x = fmaxf(x, __shfl_xor(x, 8, 64));
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

// bf16 (nearest-even) bits of a finite float.
__device__ __forceinline__ uint32_t bf16_rne(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ void __launch_bounds__(kThreads) mla_split_kernel(MlaArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t latK[kChunk * kLatPitch];
    __shared__ __attribute__((aligned(16))) uint8_t ropeK[kChunk * kRopePitch];
    __shared__ __attribute__((aligned(16))) uint8_t latT[kDc * kTPitch];
    __shared__ __attribute__((aligned(16))) uint16_t pt[kWaves][16 * kChunk];
    __shared__ int32_t sidx[kSplit];
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
    const int split = blockIdx.x, half = blockIdx.y, b = blockIdx.z;
    const int h0 = half * kHeadsPerBlock + wave * 16;          // this wave's first head
    const int k0 = split * kSplit;
    const int nk = min(kSplit, a.n_idx - k0);                  // >= 1 by the grid
    const int r16 = lane & 15, g4 = lane >> 4;

    // This split's slice of the index list; unused or out-of-range entries become -1.
    for (int i = tid; i < kSplit; i += kThreads) {
        int v = i < nk ? a.idx[(int64_t)b * a.n_idx + k0 + i] : -1;
        sidx[i] = (v >= 0 && v < a.cap) ? v : -1;
    }
    // Query fragments: A operand of K-step k (features 32k .. 32k+31; k >= 16: rotary).
    bf16x8 qa[18];
    {
        const uint16_t *ql = a.q_lat + ((int64_t)b * kH + h0 + r16) * kDc;
        const uint16_t *qr = a.q_rope + ((int64_t)b * kH + h0 + r16) * kDr;
#pragma unroll
        for (int k = 0; k < 16; k++) qa[k] = as_bf16x8(*reinterpret_cast<const uint4 *>(ql + 32 * k + 8 * g4));
#pragma unroll
        for (int k = 0; k < 2; k++) qa[16 + k] = as_bf16x8(*reinterpret_cast<const uint4 *>(qr + 32 * k + 8 * g4));
    }
    f32x4 o[kDc / 16];
#pragma unroll
    for (int n = 0; n < kDc / 16; n++) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[4], l[4];                                          // heads 4 * g4 + i of this wave
#pragma unroll
    for (int i = 0; i < 4; i++) {
        m[i] = -__builtin_inff();
        l[i] = 0.f;
    }
    const float sl2 = a.scale * 1.4426950408889634f;           // logits in base-2 units
    __syncthreads();

    const int nchunks = (nk + kChunk - 1) / kChunk;
    const int fg = tid & 63, kg = tid >> 6;                    // staging tile: features 8fg.., keys 8kg..
    for (int c = 0; c < nchunks; c++) {
        // ---- gather the chunk: latent (one 8 x 8 tile per thread) and rotary rows
        {
            uint4 v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int row = sidx[c * kChunk + 8 * kg + j];
                const int64_t r = row < 0 ? 0 : row;
                v[j] = *reinterpret_cast<const uint4 *>(a.kv_lat + ((int64_t)b * a.stride + r) * kDc + 8 * fg);
            }
            const int rk = tid >> 3, rp = tid & 7;             // rotary: key rk, 16-byte part rp
            const int rrow = sidx[c * kChunk + rk];
            const uint4 rv = *reinterpret_cast<const uint4 *>(
                a.kv_rope + ((int64_t)b * a.stride + (rrow < 0 ? 0 : rrow)) * kDr + 8 * rp);
#pragma unroll
            for (int j = 0; j < 8; j++) *reinterpret_cast<uint4 *>(latK + (8 * kg + j) * kLatPitch + 16 * fg) = v[j];
            *reinterpret_cast<uint4 *>(ropeK + rk * kRopePitch + 16 * rp) = rv;
            // transpose: w holds keys 8kg .. 8kg+7 of feature 8fg + f (dword d of v[j] holds
            // features 2d and 2d + 1 of key 8kg + j)
#pragma unroll
            for (int f = 0; f < 8; f++) {
                uint32_t w[4];
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const uint32_t lo = dword_of(v[2 * jj], f / 2), hi = dword_of(v[2 * jj + 1], f / 2);
                    // bf16 f of key 2jj (low half) and of key 2jj+1 (high half)
                    w[jj] = (f & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
                }
                *reinterpret_cast<uint4 *>(latT + (8 * fg + f) * kTPitch + 16 * kg) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        __syncthreads();
        // ---- S = Q K^T: 16 heads x 32 keys (two 16 x 16 tiles)
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 18; k++) {
            uint4 b0, b1;
            if (k < 16) {
                b0 = *reinterpret_cast<const uint4 *>(latK + r16 * kLatPitch + 64 * k + 16 * g4);
                b1 = *reinterpret_cast<const uint4 *>(latK + (16 + r16) * kLatPitch + 64 * k + 16 * g4);
            } else {
                b0 = *reinterpret_cast<const uint4 *>(ropeK + r16 * kRopePitch + 64 * (k - 16) + 16 * g4);
                b1 = *reinterpret_cast<const uint4 *>(ropeK + (16 + r16) * kRopePitch + 64 * (k - 16) + 16 * g4);
            }
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], as_bf16x8(b0), s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], as_bf16x8(b1), s1, 0, 0, 0);
        }
        // lane holds keys r16 (s0) and 16 + r16 (s1) of heads 4 g4 + i
        const bool ok0 = sidx[c * kChunk + r16] >= 0, ok1 = sidx[c * kChunk + 16 + r16] >= 0;
        float alpha[4];
        bool rescale = false;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float x0 = ok0 ? s0[i] * sl2 : -__builtin_inff();
            const float x1 = ok1 ? s1[i] * sl2 : -__builtin_inff();
            const float mn = fmaxf(m[i], row16_max(fmaxf(x0, x1)));
            float p0 = 0.f, p1 = 0.f;
            alpha[i] = 1.f;
            if (mn != -__builtin_inff()) {
                alpha[i] = exp2f(m[i] - mn);                   // 0 when m was -inf
                p0 = exp2f(x0 - mn);
                p1 = exp2f(x1 - mn);
            }
            const uint32_t q0 = bf16_rne(p0), q1 = bf16_rne(p1);
            l[i] = l[i] * alpha[i] + row16_sum(__uint_as_float(q0 << 16) + __uint_as_float(q1 << 16));
            m[i] = mn;
            rescale |= alpha[i] != 1.f;
            pt[wave][(4 * g4 + i) * kChunk + r16] = (uint16_t)q0;
            pt[wave][(4 * g4 + i) * kChunk + 16 + r16] = (uint16_t)q1;
        }
        if (__any(rescale)) {
#pragma unroll
            for (int n = 0; n < kDc / 16; n++)
#pragma unroll
                for (int i = 0; i < 4; i++) o[n][i] *= alpha[i];
        }
        // ---- O += P V: A = P (16 heads x 32 keys), B = V (32 keys x 16 features) per tile
        const bf16x8 pa = as_bf16x8(*reinterpret_cast<const uint4 *>(&pt[wave][r16 * kChunk + 8 * g4]));
#pragma unroll
        for (int n = 0; n < kDc / 16; n++) {
            const uint4 vb = *reinterpret_cast<const uint4 *>(latT + (16 * n + r16) * kTPitch + 16 * g4);
            o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(vb), o[n], 0, 0, 0);
        }
        __syncthreads();                                       // before the next gather overwrites LDS
    }
    // ---- partials: unnormalised o, running max (base-2 units) and sum per head
    float *op = a.o_part + (((int64_t)b * a.nsplit + split) * kH + h0) * kDc;
#pragma unroll
    for (int n = 0; n < kDc / 16; n++)
#pragma unroll
        for (int i = 0; i < 4; i++) op[(int64_t)(4 * g4 + i) * kDc + 16 * n + r16] = o[n][i];
    if (r16 == 0) {
        float *mp = a.ml_part + (((int64_t)b * a.nsplit + split) * kH + h0) * 2;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            mp[2 * (4 * g4 + i)] = m[i];
            mp[2 * (4 * g4 + i) + 1] = l[i];
        }
    }
}

// One block per (b, head): 256 threads x 2 features.
__global__ void __launch_bounds__(256) mla_combine_kernel(MlaArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    float M = -__builtin_inff();
    for (int s = 0; s < a.nsplit; s++) {
        const float ms = a.ml_part[(((int64_t)b * a.nsplit + s) * kH + h) * 2];
        M = fmaxf(M, ms);
    }
    float den = 0.f, acc0 = 0.f, acc1 = 0.f;
    const int c = 2 * threadIdx.x;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < a.nsplit; s++) {
            const float *ml = a.ml_part + (((int64_t)b * a.nsplit + s) * kH + h) * 2;
            const float ms = ml[0];
            if (ms == -__builtin_inff()) continue;
            const float wgt = exp2f(ms - M);
            den += wgt * ml[1];
            const float2 v = *reinterpret_cast<const float2 *>(a.o_part + (((int64_t)b * a.nsplit + s) * kH + h) * kDc + c);
            acc0 += wgt * v.x;
            acc1 += wgt * v.y;
        }
    }
    float2 r = make_float2(0.f, 0.f);
    if (den > 0.f) r = make_float2(acc0 / den, acc1 / den);
    *reinterpret_cast<float2 *>(a.out + ((int64_t)b * kH + h) * kDc + c) = r;
}

}  // namespace

size_t mla_workspace_bytes(int32_t B, int32_t n_idx) {
    const int64_t nsplit = (n_idx + kSplit - 1) / kSplit;
    return (size_t)B * nsplit * kH * (kDc + 2) * sizeof(float);
}

hipError_t launch_sparse_mla(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *kv_lat,
                             const uint16_t *kv_rope, int64_t stride, int64_t cap, const int32_t *idx, int32_t B,
                             int32_t n_idx, float scale, float *out, void *workspace, hipStream_t stream) {
    MlaArgs a{};
    a.q_lat = q_lat;
    a.q_rope = q_rope;
    a.kv_lat = kv_lat;
    a.kv_rope = kv_rope;
    a.stride = stride;
    a.cap = cap;
    a.idx = idx;
    a.n_idx = n_idx;
    a.nsplit = (n_idx + kSplit - 1) / kSplit;
    a.scale = scale;
    a.o_part = static_cast<float *>(workspace);
    a.ml_part = a.o_part + (int64_t)B * a.nsplit * kH * kDc;
    a.out = out;
    if (a.nsplit > 0) {
        hipError_t e = launch(mla_split_kernel, dim3((unsigned)a.nsplit, kH / kHeadsPerBlock, (unsigned)B),
                              dim3(kThreads), 0u, stream, a);
        if (e != hipSuccess) return e;
    }
    return launch(mla_combine_kernel, dim3(kH, (unsigned)B), dim3(kDc / 2), 0u, stream, a);
}

}  // namespace lk

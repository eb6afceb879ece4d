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
// A chunk's latent (1 KB) and rotary (128 B) rows are gathered from HBM straight into
// LDS by DMA (global_load_lds: one instruction moves one latent row, or eight rotary
// rows), key-major, with each row's 16-byte chunks XOR-swizzled by the row index
// through the source address.  Two chunk buffers alternate: the DMA of chunk c+1 is
// in flight while chunk c is computed.  Each wave keeps its 16 heads' query (576
// features, bf16) in registers as the A operand of v_mfma_f32_16x16x32_bf16 for
// S = Q K^T; the P V product takes its B operand (8 consecutive keys of one latent
// feature per lane) from the same key-major rows with two transposing LDS reads
// (ds_read_b64_tr_b16: within 16 lanes, lane l receives element l % 4 of the 8-byte
// pieces read by lanes 4i + l / 4).  Online softmax per wave (row max and sum over
// the 16 lanes that hold one head's keys); p rounded to bf16 for P V; o for 16 heads
// x 512 features accumulates in 128 registers per lane.  The split writes its
// unnormalised o with the running max m and sum l to the workspace.
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
constexpr int kLatRow = 2 * kDc;               // bytes per latent row in LDS (64 chunks of 16 B)
constexpr int kRopeRow = 2 * kDr;             // bytes per rotary row in LDS (8 chunks of 16 B)
static_assert(kThreads == 2 * 4 * kChunk, "8 lanes x 4 waves per 32-key chunk row set");

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

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

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

// One 16-byte-per-lane DMA from global memory into LDS at lds + 16 * lane.  Written as
// inline asm so that the compiler does not make later LDS reads wait for it (it cannot
// tell the two chunk buffers apart); the caller waits with vmcnt before the barrier
// that publishes the data.  M0 holds the LDS base; an LDS DMA needs one wait state
// after M0 is written.
__device__ __forceinline__ void dma16(const void *src, const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}

// Gather chunk c (keys sidx[32c .. 32c+31]) into lat / rope: wave w moves latent rows
// 8w .. 8w+7 (one DMA each) and rotary rows 8w .. 8w+7 (one DMA).  Row r's 16-byte
// chunk j lands in slot j ^ (r % 16) (latent) or j ^ (r % 8) (rotary).
__device__ __forceinline__ void gather_chunk(const MlaArgs &a, int b, const int32_t *sidx, int c, uint8_t *lat,
                                             uint8_t *rope, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int r = 8 * wave + j;
        const int row = sidx[c * kChunk + r];
        const int64_t g = (int64_t)b * a.stride + (row < 0 ? 0 : row);
        const uint8_t *src = reinterpret_cast<const uint8_t *>(a.kv_lat) + g * kLatRow + 16 * (lane ^ (r & 15));
        dma16(src, lat + r * kLatRow);
    }
    const int r = 8 * wave + (lane >> 3);
    const int row = sidx[c * kChunk + r];
    const int64_t g = (int64_t)b * a.stride + (row < 0 ? 0 : row);
    const uint8_t *src = reinterpret_cast<const uint8_t *>(a.kv_rope) + g * kRopeRow + 16 * ((lane & 7) ^ (r & 7));
    dma16(src, rope + 8 * wave * kRopeRow);
}

// Per-lane LDS byte offsets of the swizzled rows, fixed for the whole kernel.  Every
// read below is one of these plus a constant: XOR with the row index only touches the
// low four bits of a 16-byte chunk number, so chunk 16 j + c' of a row lies 256 j
// bytes after chunk c'.
struct LdsOffsets {
    uint32_t s_lat[4];       // S: latent row r16, chunk 4 kk + g4 (kk = k % 4)
    uint32_t s_rope[2];      // S: rotary row r16, chunk 4 kk + g4
    uint32_t pv[2][8];       // P V: transposing read h, feature chunk pair n' (n = 8 j + n')
};

__device__ __forceinline__ LdsOffsets lds_offsets(int lane) {
    const int r16 = lane & 15, g4 = lane >> 4, sq = r16 & 3;
    LdsOffsets t;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) t.s_lat[kk] = r16 * kLatRow + 16 * ((4 * kk + g4) ^ r16);
#pragma unroll
    for (int kk = 0; kk < 2; kk++) t.s_rope[kk] = r16 * kRopeRow + 16 * ((4 * kk + g4) ^ (r16 & 7));
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int row = 8 * g4 + 4 * h + (r16 >> 2);
#pragma unroll
        for (int n = 0; n < 8; n++) t.pv[h][n] = row * kLatRow + 16 * ((2 * n + (sq >> 1)) ^ (row & 15)) + 8 * (sq & 1);
    }
    return t;
}

// Raise the running max only when a chunk exceeds it by more than 2^8 (base-2 logits):
// p = 2^(x - m) then stays below 2^8, and the rescale of o (128 registers) runs on
// few chunks.  The result does not depend on which m is used.
constexpr float kLazyMax = 8.f;

// One chunk of S = Q K^T, online softmax and O += P V for this wave's 16 heads.
__device__ __forceinline__ void chunk_compute(const bf16x8 qa[18], const uint8_t *lat, const uint8_t *rope,
                                              const LdsOffsets &off, const int32_t *sidx, int c, float sl2,
                                              float m[4], float l[4], f32x4 o[kDc / 16], uint16_t *ptw, int lane) {
    const int r16 = lane & 15, g4 = lane >> 4;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 18; k++) {
        const uint8_t *p0 = k < 16 ? lat + off.s_lat[k % 4] + 256 * (k / 4) : rope + off.s_rope[k - 16];
        const int second = k < 16 ? 16 * kLatRow : 16 * kRopeRow;
        const uint4 b0 = *reinterpret_cast<const uint4 *>(p0);
        const uint4 b1 = *reinterpret_cast<const uint4 *>(p0 + second);
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
        const float cm = row16_max(fmaxf(x0, x1));
        alpha[i] = 1.f;
        if (cm > m[i] + kLazyMax) {                            // also when m is -inf and cm is finite
            alpha[i] = exp2f(m[i] - cm);                       // 0 when m was -inf
            m[i] = cm;
            rescale = true;
        }
        float p0 = 0.f, p1 = 0.f;
        if (m[i] != -__builtin_inff()) {
            p0 = exp2f(x0 - m[i]);
            p1 = exp2f(x1 - m[i]);
        }
        const uint32_t q0 = bf16_rne(p0), q1 = bf16_rne(p1);
        l[i] = l[i] * alpha[i] + row16_sum(__uint_as_float(q0 << 16) + __uint_as_float(q1 << 16));
        ptw[(4 * g4 + i) * kChunk + r16] = (uint16_t)q0;
        ptw[(4 * g4 + i) * kChunk + 16 + r16] = (uint16_t)q1;
    }
    if (__any(rescale)) {
#pragma unroll
        for (int n = 0; n < kDc / 16; n++)
#pragma unroll
            for (int i = 0; i < 4; i++) o[n][i] *= alpha[i];
    }
    // O += P V.  A = P (lane: head r16, keys 8 g4 .. 8 g4 + 7).  B for tile n: keys
    // 8 g4 + 4h + i of feature 16 n + r16, from transposing reads in which source
    // lane r16 of this 16-lane group points at row 8 g4 + 4h + r16 / 4, features
    // 16 n + 4 (r16 % 4) .. + 3.
    const bf16x8 pa = as_bf16x8(*reinterpret_cast<const uint4 *>(ptw + r16 * kChunk + 8 * g4));
#pragma unroll
    for (int n = 0; n < kDc / 16; n++) {
        v4i16 half[2];
#pragma unroll
        for (int h = 0; h < 2; h++)
            half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lptr_t)(lat + off.pv[h][n % 8] + 256 * (n / 8)));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[n], 0, 0, 0);
    }
}

__global__ void __launch_bounds__(kThreads) mla_split_kernel(MlaArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lat[2][kChunk * kLatRow];
    __shared__ __attribute__((aligned(16))) uint8_t rope[2][kChunk * kRopeRow];
    __shared__ __attribute__((aligned(16))) uint16_t pt[kWaves][16 * kChunk];
    __shared__ int32_t sidx[kSplit];
    const int tid = threadIdx.x, lane = __lane_id(), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    __syncthreads();                                           // sidx

    const int nchunks = (nk + kChunk - 1) / kChunk;
    const LdsOffsets off = lds_offsets(lane);
    // One barrier per chunk: it finds chunk c's DMA landed (each wave waits for its own
    // before it) and every wave done with chunk c - 1, whose buffer then takes chunk c + 1.
    // One barrier per chunk: before it each wave waits for its own DMAs of chunk c, after
    // it every wave is done with chunk c - 1, whose buffer then takes chunk c + 1.
    gather_chunk(a, b, sidx, 0, lat[0], rope[0], wave, lane);
    for (int c = 0; c < nchunks; c++) {
        const int cur = c & 1;
        __builtin_amdgcn_s_waitcnt(0x3F70);                    // vmcnt(0): chunk c is in LDS
        __syncthreads();
        if (c + 1 < nchunks) gather_chunk(a, b, sidx, c + 1, lat[cur ^ 1], rope[cur ^ 1], wave, lane);
        chunk_compute(qa, lat[cur], rope[cur], off, sidx, c, sl2, m, l, o, pt[wave], lane);
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

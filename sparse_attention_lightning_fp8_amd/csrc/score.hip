// score.hip -- fp8 index score + mask for the lightning indexer (gfx950).
//
// Page "Index scores": S[t,s] = sum_h w[t,h] ReLU(Qbar[h,t] . kbar[s]) / (sqrt 64 sqrt 128);
// the fp8_index docstring computes it as fp8 q @ fp8 k -> fp32 logits, ReLU, times the
// folded weights, head sum, times the e8m0 key scale.  Indexer.forward then adds the
// mask (-inf outside each row's valid prefix).
//
// The contraction Q[64 x 128] x K^T[128 x keys] runs on v_mfma_f32_32x32x16_f16 with
// the e4m3fn bytes converted exactly to f16 in registers (v_cvt_scalef32_pk_f16_fp8,
// scale 1): the fp8 MFMA of gfx950 sums each group of products at reduced width and
// misses the 1e-5 relative accuracy this path is held to, while every e4m3fn value
// is an f16 normal and every f16 product is exact in the float32 accumulator.
//
// Operand layout (one wave, 32x32x16 f16): lane l supplies row (l % 32) of A (a head)
// and column (l % 32) of B (a key); lanes 0-31 carry bytes [0, 64) of the 128-byte row
// and lanes 32-63 bytes [64, 128), 8 bytes per K-step, so K-step kk pairs features
// 8kk..8kk+7 and 64+8kk..64+8kk+7 of both operands.  The accumulator of M-tile m
// (heads 32m..32m+31) holds, in lane l, key (l % 32) and heads
// 32m + 8(i/4) + 4(l/32) + (i%4) for i < 16, so a lane sums 32 heads in registers and
// one cross-half swap (v_permlane32_swap) completes the 64-head sum.
#include <type_traits>

#include "lk_device.h"
#include "quant_device.h"
#include "topk_device.h"

namespace lk {
namespace {

// Per-lane A operand (64 heads x 128 features of one query token) as f16, and the
// matching folded weights: a[m][kk] is the K-step kk operand of M-tile m.
struct QueryFrag {
    half8 a[2][8];
    float w[2][16];
};

struct QueryRaw {          // the same data before conversion (issued as early loads)
    uint4 q[2][4];
    float4 w[2][4];
};

__device__ __forceinline__ void load_query_raw(const uint8_t *__restrict__ q_row /*64 x 128*/,
                                               const float *__restrict__ w_row /*64*/, int lane,
                                               QueryRaw &raw) {
    const int r = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const uint4 *src = reinterpret_cast<const uint4 *>(q_row + (32 * m + r) * LK_DIM + 64 * hh);
#pragma unroll
        for (int c = 0; c < 4; c++) raw.q[m][c] = src[c];
#pragma unroll
        for (int g = 0; g < 4; g++) raw.w[m][g] = *reinterpret_cast<const float4 *>(w_row + 32 * m + 8 * g + 4 * hh);
    }
}

__device__ __forceinline__ void convert_query(const QueryRaw &raw, QueryFrag &f) {
#pragma unroll
    for (int m = 0; m < 2; m++) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            f.a[m][2 * c] = fp8x8_to_half8(raw.q[m][c].x, raw.q[m][c].y);
            f.a[m][2 * c + 1] = fp8x8_to_half8(raw.q[m][c].z, raw.q[m][c].w);
        }
#pragma unroll
        for (int g = 0; g < 4; g++) {
            f.w[m][4 * g + 0] = raw.w[m][g].x;
            f.w[m][4 * g + 1] = raw.w[m][g].y;
            f.w[m][4 * g + 2] = raw.w[m][g].z;
            f.w[m][4 * g + 3] = raw.w[m][g].w;
        }
    }
}

__device__ __forceinline__ void load_query(const uint8_t *__restrict__ q_row, const float *__restrict__ w_row,
                                           int lane, QueryFrag &f) {
    QueryRaw raw;
    load_query_raw(q_row, w_row, lane, raw);
    convert_query(raw, f);
}

// Head-weighted ReLU sum of the two M-tile accumulators (this lane's 32 heads).
// Scores are finite by contract, so ReLU is a single v_max (the file is built
// without NaN semantics).
__device__ __forceinline__ float relu_weighted_sum(const float16v acc[2], const QueryFrag &f) {
    // Four independent partial sums, so consecutive FMAs do not wait on each other.
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
        for (int i = 0; i < 16; i++) s[i & 3] = __builtin_fmaf(__builtin_fmaxf(acc[m][i], 0.0f), f.w[m][i], s[i & 3]);
    return (s[0] + s[1]) + (s[2] + s[3]);
}

// The 16 MFMAs of one 32-key tile whose B operand (this lane's 64 bytes of key l % 32)
// is `kv`: acc[m] holds heads 32m .. 32m + 31 against the tile's keys.  Each fp8 K-step
// is converted to f16 right before its two MFMAs.
__device__ __forceinline__ void mfma_tile(const uint4 (&kv)[4], const QueryFrag &f, float16v (&acc)[2]) {
    acc[0] = float16v{};
    acc[1] = float16v{};
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const half8 b0 = fp8x8_to_half8(kv[c].x, kv[c].y);
        const half8 b1 = fp8x8_to_half8(kv[c].z, kv[c].w);
#pragma unroll
        for (int m = 0; m < 2; m++) {
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[m][2 * c], b0, acc[m], 0, 0, 0);
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[m][2 * c + 1], b1, acc[m], 0, 0, 0);
        }
    }
}

// One wave's kTiles tiles of 32 consecutive keys from key0, as a software pipeline:
// step j issues the MFMAs of tile j + 1 interleaved with the ReLU / weight / head-sum
// epilogue of tile j, so with one or two waves per SIMD the matrix core and the VALU
// still overlap.  Tiles 0 .. kFly - 1 must be in flight already; step j issues tile
// j + kFly (load_tile(j + kFly)), kFly steps before it is needed.  Two tiles make 64
// keys, one per lane after a cross-half swap (lanes 0-31: tile 2p, lanes 32-63: tile
// 2p + 1 -> key key0 + 64 p + lane), scaled by ks[p] and stored (-inf past the valid
// prefix L, nothing past T).
template <int kTiles, int kFly, typename LoadTile>
__device__ __forceinline__ void pipelined_tiles(uint4 (&kv)[kTiles][4], LoadTile load_tile, const QueryFrag &f,
                                                const float (&ks)[kTiles / 2], int64_t key0, int64_t T, int64_t L,
                                                float *out) {
    static_assert(kTiles % 2 == 0 && kFly >= 1 && kFly <= kTiles, "tile schedule");
    const int lane = __lane_id();
    auto start_tile = [&](int j, float16v (&acc)[2]) { mfma_tile(kv[j], f, acc); };
    float16v acc[2][2];
    float part[2];
    start_tile(0, acc[0]);
#pragma unroll
    for (int j = 0; j < kTiles; j++) {
        __builtin_amdgcn_sched_barrier(0);
        if (j + kFly < kTiles) load_tile(j + kFly);
        if (j + 1 < kTiles) start_tile(j + 1, acc[(j + 1) & 1]);
        part[j & 1] = relu_weighted_sum(acc[j & 1], f);
        if (j & 1) {
            const float sum = halves_sum_pair(part[0], part[1]);
            const int64_t s = key0 + 64 * (j / 2) + lane;
            if (s < T) out[s] = s < L ? sum * ks[j / 2] : -__builtin_inff();
        }
        if (j + 1 < kTiles) {
#pragma unroll
            for (int c = 0; c < 8; c++) {
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // conversions of the next K-step
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // its two MFMAs
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // epilogue VALU of the current tile
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------ decode (S == 1)
// Work is cut into items of kDecKeysPerBlock (1024) consecutive keys of one query row.
// Four kernels cover them:
//  - decode_kernel (the fused step, one block per item): loader waves stream the
//    item's keys into LDS while compute waves prepare the query; as
//    decode_kernel<true> (lk_decode_select, rows of one item) the block also keeps
//    its scores in LDS and its loader waves then select the row's top-k from there;
//  - decode_units_kernel (when the items outnumber what the chip runs at once, for the
//    fused step and for lk_index_score alike): the same loader-wave block over a
//    balanced run of 512-key units of one row, one per compute unit; the standalone
//    form reads the prepared query instead of quantizing it and writes no key;
//  - decode_pipe_kernel (lk_index_score with a prepared query, one block per item):
//    four waves with K in registers.
//
// The fused kernels (lk_decode_score) start from the bf16 query, the raw weights and
// the new key of the decode step: each block quantizes the row's 64 query heads itself
// (8 lanes per head, the same arithmetic as lk_quantize_queries), and the block
// holding key L-1 (the new token's slot) also rotates and quantizes the new key,
// writes it to the cache, and hands it to the lanes that score it in place of the
// stale cache row they loaded.
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecTiles = 4;                       // 32-key tiles per wave
constexpr int kDecKeysPerWave = 32 * kDecTiles;    // 128
constexpr int kDecKeysPerBlock = kDecKeysPerWave * kDecWaves;
constexpr int kQPitch = LK_DIM + 16;               // LDS row pitch of the staged query (spreads banks)
static_assert(LK_HEADS * LK_DIM / 16 == kDecThreads, "one 16-byte query piece per thread");
static_assert(LK_HEADS * 8 == kDecThreads, "one 8-lane row group per head");

struct DecodeArgs {
    const uint8_t *q_fp8;       // [B, 64, 128] e4m3fn        (standalone score)
    const float *w_eff;         // [B, 64] folded weights     (standalone score)
    const uint16_t *q_bf16;     // [B, 64, 128] bf16          (fused)
    const float *w;             // [B, 64] raw weights        (fused)
    const uint16_t *k_new;      // [B, 128] bf16 new keys     (fused)
    uint8_t *q_fp8_out;         // optional copies of the quantized query (fused)
    float *w_eff_out;
    const float *rope_cos;      // optional [B][32] RoPE tables of the step's token (fused)
    const float *rope_sin;
    uint8_t *k_cache;           // [B, stride, 128]; the fused kernel writes row L-1
    float *k_scale;             // [B, stride]
    int64_t cache_seq_stride;
    RowsDev rows;
    float *scores;              // [B, T]; may be NULL in the fused select kernel
    int32_t k;                  // fused select: the top-k of each row into idx [B, k]
    int32_t *idx;
};

struct DecodeShared {
    uint8_t sq[LK_HEADS * kQPitch];             // the row's quantized query (A operand source)
    float sw[LK_HEADS];                         // its folded weights
    uint4 snew[8];                              // fused: the new key's 128 codes
    float snew_scale;
};

// ------------------------------------------------------------------ decode, fused step
// One block per item, K streamed into LDS by dedicated waves.  A wave that issues
// loads stalls once the compute unit's memory queue is full (it drains at the chip's
// HBM rate), so with K loaded into each wave's own registers every wave
// waits behind its K loads before it can start the query preparation, which the whole
// item then waits for.  Here four loader waves move the item's 1024 keys (128 KB)
// into LDS with global_load_lds DMA, in four phases of 32 KB (phase p = tile p of
// every compute wave), while the eight compute waves issue only their small loads,
// prepare the query at once, and then take each phase from LDS behind one block
// barrier per phase (12 waves, 3 per SIMD, so the epilogue reads the folded weights
// from LDS instead of holding them in registers).
// LDS layout of a phase: the 8 compute waves' tiles of 32 rows x 128 B, rows in key
// order; the 16-byte chunk q of a tile's row r sits in slot q ^ ((r >> 1) & 7), so the
// MFMA B-operand reads (lanes 0-31 rows 0-31, 16 bytes each) touch every bank once per
// 16 lanes.  A DMA instruction writes 1 KB = 8 consecutive rows, lane i filling slot
// i % 8 of row i / 8 with the chunk that belongs there.
constexpr int kDmaComputeWaves = kDecWaves;
constexpr int kDmaLoaderWaves = 4;
constexpr int kDmaThreads = 64 * (kDmaComputeWaves + kDmaLoaderWaves);
constexpr int kDmaPhaseBytes = kDmaComputeWaves * 32 * LK_DIM;            // 32 KB
constexpr int kDmaPerPhase = kDmaPhaseBytes / 1024 / kDmaLoaderWaves;     // DMA instructions per loader wave
static_assert(kDmaPerPhase * kDmaLoaderWaves * 1024 == kDmaPhaseBytes, "phase split");

struct DmaShared {
    uint8_t k[kDecTiles * kDmaPhaseBytes];
    DecodeShared d;
};

// Fused select (rows of at most one key block): the block's scores, then the row's
// top-k run by the loader waves once the compute waves are done.
struct SelectShared {
    float sc[kDecKeysPerBlock] __attribute__((aligned(16)));
    TopkShared<64 * kDmaLoaderWaves> t;
};
static_assert(64 * kDmaLoaderWaves == 256 && Shape<256>::kMaxT >= kDecKeysPerBlock, "the loader waves' top-k shape");

__device__ __forceinline__ int kslot(int r, int q) { return q ^ ((r >> 1) & 7); }

template <bool kSelect>
__global__ void __launch_bounds__(kDmaThreads) decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) DmaShared sm;
    __shared__ std::conditional_t<kSelect, SelectShared, char> ssel;
    LK_POISON_LDS_OBJS(sm, ssel);
    uint8_t *const sq = sm.d.sq;
    float *const sw = sm.d.sw;
    uint4 *const snew = sm.d.snew;
    const int qrow = blockIdx.y;
    const int64_t blk0 = (int64_t)blockIdx.x * kDecKeysPerBlock;
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
    const int b = qrow / a.rows.S;
    const int t = qrow - b * a.rows.S;
    const int64_t T = a.rows.T;
    const int64_t L = row_len(a.rows, b, t);
    float *out = a.scores ? a.scores + (int64_t)qrow * T : nullptr;   // NULL only in the fused select
    const bool loader = wave >= kDmaComputeWaves;
    const int head = threadIdx.x >> 3, sub = threadIdx.x & 7;   // compute waves: this thread's 16 features of a head
    const bool rope_on = a.rope_cos != nullptr;
    // The fused select may leave the scores out; the select kernel has one block per row.
    const bool keep_scores = !kSelect || a.scores != nullptr;
    if (blk0 >= L) {                                   // the whole block is masked: -inf only
        if (loader) return;
        if (keep_scores)
            for (int64_t s = blk0 + threadIdx.x; s < blk0 + kDecKeysPerBlock && s < T; s += 64 * kDmaComputeWaves)
                out[s] = -__builtin_inff();
        if constexpr (kSelect)                         // L == 0: nothing is selected
            for (int j = threadIdx.x; j < a.k; j += 64 * kDmaComputeWaves) a.idx[(int64_t)qrow * a.k + j] = -1;
        if (blk0 == 0 && a.q_fp8_out) {                // a row with L == 0 still returns its quantized query
            const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_bf16 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
            const uint4 q0 = qs[0], q1 = qs[1];
            uint32_t in[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            if (rope_on) {
                Rope16 rr;
                load_rope16(a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2), a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2), sub, rr);
                rope_row16(in, rr, sub);
            }
            uint32_t codes[4];
            int j;
            quantize_row16(in, codes, j);
            *reinterpret_cast<uint4 *>(a.q_fp8_out + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub) =
                make_uint4(codes[0], codes[1], codes[2], codes[3]);
            if (sub == 0) a.w_eff_out[(int64_t)qrow * LK_HEADS + head] = fold_weight(a.w[(int64_t)qrow * LK_HEADS + head], j);
        }
        return;
    }
    const uint8_t *kbase = a.k_cache + (int64_t)b * a.cache_seq_stride * LK_DIM;
    if (loader) {
        // Loader wave v: in phase p, DMA instruction i covers phase rows 8 (v * kDmaPerPhase + i) .. +7.
        const int v = wave - kDmaComputeWaves;
        auto issue_phase = [&](int p) {
#pragma unroll
            for (int i = 0; i < kDmaPerPhase; i++) {
                const int R = 8 * (v * kDmaPerPhase + i) + (lane >> 3);   // row within the phase
                const int w = R >> 5, r = R & 31;
                const int q = kslot(r, lane & 7);                         // the chunk this lane's slot holds
                const int64_t s = blk0 + 32 * (kDecTiles * w + p) + r;
                const uint8_t *src = kbase + (s < L ? s : 0) * LK_DIM + 16 * q;
                dma_b128(src, sm.k + p * kDmaPhaseBytes + 1024 * (v * kDmaPerPhase + i));
            }
        };
        // Two phases in flight: issuing all four at once keeps these waves in their
        // issue loop until half the block has landed, and the first barrier waits
        // for them (measured slower).
        issue_phase(0);
        issue_phase(1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerPhase));
        __syncthreads();                               // phase 0 landed (and the query is prepared)
        issue_phase(2);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerPhase));
        __syncthreads();                               // phase 1
        issue_phase(3);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerPhase));
        __syncthreads();                               // phase 2
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();                               // phase 3
        if constexpr (kSelect) {
            __syncthreads();                           // the block's scores are in LDS
            topk_row<64 * kDmaLoaderWaves>(ssel.sc, kDecKeysPerBlock, L, a.k, a.idx + (int64_t)qrow * a.k,
                                           (int)threadIdx.x - 64 * kDmaComputeWaves, ssel.t.view());
        }
        return;
    }

    // Compute wave `wave`: keys key0 .. key0 + 127 (its tile p is in phase p).
    const int64_t key0 = blk0 + (int64_t)wave * kDecKeysPerWave;
    const int r = lane & 31, hh = lane >> 5;
    const int64_t pn = L - 1 < blk0 + kDecKeysPerBlock ? L - 1 : -1;   // the new key's slot (uniform)
    const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_bf16 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
    const uint4 qp0 = qs[0], qp1 = qs[1];
    const float wr = a.w[(int64_t)qrow * LK_HEADS + head];
    const uint32_t kn = reinterpret_cast<const uint32_t *>(a.k_new + (int64_t)b * LK_DIM)[lane];
    const float *kc_row = rope_on ? a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2) : reinterpret_cast<const float *>(a.k_new);
    const float *ks_row = rope_on ? a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2) : reinterpret_cast<const float *>(a.k_new);
    const float2 krc = reinterpret_cast<const float2 *>(kc_row)[lane & 15];
    const float2 krs = reinterpret_cast<const float2 *>(ks_row)[lane & 15];
    Rope32 rope_row;
    if (rope_on)
        load_rope32_uniform(a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2),
                            a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2), rope_row);
    float ks[kDecTiles / 2];
#pragma unroll
    for (int p = 0; p < kDecTiles / 2; p++) {
        const int64_t s = key0 + 64 * p + lane;
        ks[p] = a.k_scale[(int64_t)b * a.cache_seq_stride + (s < L ? s : 0)];
    }
    {
        uint32_t in[8] = {qp0.x, qp0.y, qp0.z, qp0.w, qp1.x, qp1.y, qp1.z, qp1.w};
        if (rope_on) {
            Rope16 rope;
            pick_rope16(rope_row, sub, rope);
            rope_row16(in, rope, sub);
        }
        uint32_t codes[4];
        int j;
        quantize_row16(in, codes, j);
        const uint4 piece = make_uint4(codes[0], codes[1], codes[2], codes[3]);
        *reinterpret_cast<uint4 *>(sq + head * kQPitch + 16 * sub) = piece;
        const float we = fold_weight(wr, j);
        if (sub == 0) sw[head] = we;
        if (blk0 == 0 && a.q_fp8_out) {
            *reinterpret_cast<uint4 *>(a.q_fp8_out + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub) = piece;
            if (sub == 0) a.w_eff_out[(int64_t)qrow * LK_HEADS + head] = we;
        }
    }
    if (pn >= 0 && wave == 0) {                        // the new key, spread over wave 0 (2 features a lane)
        uint32_t kin = kn;
        if (rope_on) rope_row_wave(kin, krc, krs);
        int kj;
        const uint32_t kc = quantize_row_wave(kin, kj);
        const int64_t row = (int64_t)b * a.cache_seq_stride + pn;
        reinterpret_cast<uint16_t *>(a.k_cache + row * LK_DIM)[lane] = (uint16_t)kc;
        reinterpret_cast<uint16_t *>(snew)[lane] = (uint16_t)kc;
        if (lane == 0) {
            const float ksc = __builtin_ldexpf(1.0f, kj);
            a.k_scale[row] = ksc;
            sm.d.snew_scale = ksc;
        }
    }
    __syncthreads();                                   // query prepared, phase 0 landed
    QueryRaw raw;
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const uint8_t *qr = sq + (32 * m + r) * kQPitch + 64 * hh;
#pragma unroll
        for (int c = 0; c < 4; c++) raw.q[m][c] = *reinterpret_cast<const uint4 *>(qr + 16 * c);
#pragma unroll
        for (int g = 0; g < 4; g++) raw.w[m][g] = *reinterpret_cast<const float4 *>(sw + 32 * m + 8 * g + 4 * hh);
    }
    QueryFrag f;
    convert_query(raw, f);
    // relu_weighted_sum with the weights read from LDS, in the same order.
    // The weight quads are read two at a time: one at a time, the register budget made
    // the compiler wait out each LDS read before the next (eight round trips per tile).
    auto relu_weighted_sum_lds = [&](const float16v (&acc2)[2]) {
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i0 = 0; i0 < 8; i0 += 2) {
            float4 wq[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = (i0 + i) >> 2, g = (i0 + i) & 3;
                wq[i] = *reinterpret_cast<const float4 *>(sw + 32 * m + 8 * g + 4 * hh);
            }
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = (i0 + i) >> 2, g = (i0 + i) & 3;
                const float wg[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
#pragma unroll
                for (int k = 0; k < 4; k++)
                    s4[k] = __builtin_fmaf(__builtin_fmaxf(acc2[m][4 * g + k], 0.0f), wg[k], s4[k]);
            }
        }
        return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    {
        const float nscale = sm.d.snew_scale;
#pragma unroll
        for (int p = 0; p < kDecTiles / 2; p++) ks[p] = key0 + 64 * p + lane == pn ? nscale : ks[p];
    }
    float16v acc[2][2];
    float part[2];
#pragma unroll
    for (int p = 0; p < kDecTiles; p++) {
        if (p > 0) __syncthreads();                    // phase p landed
        uint4 kv[4];
        const uint8_t *row = sm.k + p * kDmaPhaseBytes + (32 * wave + r) * LK_DIM;
#pragma unroll
        for (int c = 0; c < 4; c++) kv[c] = *reinterpret_cast<const uint4 *>(row + 16 * kslot(r, 4 * hh + c));
        const bool mine = key0 + 32 * p + r == pn;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const uint4 n = snew[4 * hh + c];
            kv[c].x = mine ? n.x : kv[c].x;
            kv[c].y = mine ? n.y : kv[c].y;
            kv[c].z = mine ? n.z : kv[c].z;
            kv[c].w = mine ? n.w : kv[c].w;
        }
        mfma_tile(kv, f, acc[p & 1]);
        if (p > 0) {
            part[(p - 1) & 1] = relu_weighted_sum_lds(acc[(p - 1) & 1]);
            if (p == 2) {
                const float sum = halves_sum_pair(part[0], part[1]);
                const int64_t s = key0 + lane;
                const float v = s < L ? sum * ks[0] : -__builtin_inff();
                if (s < T && keep_scores) out[s] = v;
                if constexpr (kSelect) ssel.sc[s - blk0] = v;
            }
        }
    }
    part[1] = relu_weighted_sum_lds(acc[1]);
    const float sum = halves_sum_pair(part[0], part[1]);
    const int64_t s = key0 + 64 + lane;
    const float v = s < L ? sum * ks[1] : -__builtin_inff();
    if (s < T && keep_scores) out[s] = v;
    if constexpr (kSelect) {
        ssel.sc[s - blk0] = v;
        __syncthreads();                               // hand the scores to the loader waves' top-k
    }
}

// ------------------------------------------------------------------ decode, fused, many items
// The fused step when the rows' 1024-key items outnumber what one wave of blocks covers
// (ragged rows among them): one loader-wave block per compute unit, each scoring a run
// of consecutive 512-key units of one row, so one query preparation serves the whole
// run.  A unit is two 32-key tiles of every compute wave (wave w takes keys 64 w .. 64 w
// + 63 of the unit); the loaders stream its two phases through the same four 32 KB
// buffers, two phases ahead, and every phase ends in one block barrier as in
// decode_kernel.  Runs never cross a row and are balanced at unit granularity: every
// block derives the same schedule from the row lengths (row r has
// u_r = max(1, ceil(L_r / 512)) units; the cap c is the smallest for which the rows'
// ceil(u_r / c) runs fit the grid; row r's units are split into that many runs of equal
// size up to one), and block g takes run g.  A row with L_r = 0 gets one empty run that
// sweeps it to -inf (and writes its quantized query when that is requested); the last
// run of every row sweeps the slots past its units.
constexpr int kUnitKeys = kDecKeysPerBlock / 2;                 // 512
constexpr int kUnitTiles = kUnitKeys / (32 * kDmaComputeWaves); // 2 tiles per compute wave
constexpr int kUnitMaxRows = kDecThreads;                         // rows the schedule takes (one per thread)
static_assert(kUnitTiles == 2 && kDecTiles == 4, "a unit is two phases of the four-buffer ring");
static_assert(kUnitMaxRows <= kDmaThreads, "one row per thread in the schedule");

struct UnitShared {
    DmaShared s;
    int64_t run_len;                                   // the row's valid length L
    int32_t run[5];                                    // this block's row, first unit, units, last, runs in all
    int32_t part[kDmaThreads / 64];                    // per-wave partial sums of the schedule
};

template <bool kFused>
__global__ void __launch_bounds__(kDmaThreads) decode_units_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) UnitShared us;
    LK_POISON_LDS_OBJS(us);
    DmaShared &sm = us.s;
    uint8_t *const sq = sm.d.sq;
    float *const sw = sm.d.sw;
    uint4 *const snew = sm.d.snew;
    const int nrows = a.rows.B;                        // S == 1; nrows <= kUnitMaxRows (host check)
    const int tid = threadIdx.x, lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // ---- the schedule (every block the same).  Up to 64 rows, wave 0 derives it with
    // lane shuffles and hands this block's run to the others through LDS (one barrier);
    // more rows take the block-wide form (one row per thread, block sums and a scan).
    const int G = gridDim.x, g = blockIdx.x;
    if (nrows <= 64) {
        if (wave == 0) {
            int64_t Lr = 0;
            int u = 0;
            if (lane < nrows) {
                Lr = row_len(a.rows, lane, 0);
                const int64_t ur = (Lr + kUnitKeys - 1) / kUnitKeys;
                u = ur < 1 ? 1 : (int)ur;
            }
            auto wave_sum = [&](int x) {
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
                return x;
            };
            int cap = (wave_sum(u) + G - 1) / G;
            for (;; cap++)                             // ends by cap = max u_r (then nrows <= G runs)
                if (wave_sum(lane < nrows ? (u + cap - 1) / cap : 0) <= G) break;
            const int nr = lane < nrows ? (u + cap - 1) / cap : 0;
            int incl = nr;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            const int first = incl - nr;
            if (lane < nrows && first <= g && g < incl) {   // the lane of this block's row
                const int k = g - first, q_u = u / nr, r_u = u % nr;
                us.run[0] = lane;
                us.run[1] = k * q_u + (k < r_u ? k : r_u);  // first unit
                us.run[2] = q_u + (k < r_u ? 1 : 0);        // units
                us.run[3] = k == nr - 1;                    // the row's last run
                us.run_len = Lr;
            }
            if (lane == 63) us.run[4] = incl;               // runs in all
        }
        __syncthreads();
    } else {
        int64_t Lr = 0;
        int u = 0;
        if (tid < nrows) {
            Lr = row_len(a.rows, tid, 0);
            const int64_t ur = (Lr + kUnitKeys - 1) / kUnitKeys;
            u = ur < 1 ? 1 : (int)ur;
        }
        auto block_sum = [&](int x) {                  // block sum of x (uniform result)
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
            __syncthreads();                           // earlier readers of us.part are done
            if (lane == 0) us.part[wave] = x;
            __syncthreads();
            int t = 0;
#pragma unroll
            for (int w = 0; w < kDmaThreads / 64; w++) t += us.part[w];
            return t;
        };
        int cap = (block_sum(u) + G - 1) / G;
        for (;; cap++) {                               // ends by cap = max u_r (then nrows <= G runs)
            const int n = tid < nrows ? (u + cap - 1) / cap : 0;
            if (block_sum(n) <= G) break;
        }
        const int nr = tid < nrows ? (u + cap - 1) / cap : 0;   // this row's runs
        int incl = nr;                                 // inclusive scan of nr over the rows
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (lane >= d) incl += y;
        }
        __syncthreads();
        if (lane == 63) us.part[wave] = incl;
        __syncthreads();
        int base = 0;
#pragma unroll
        for (int w = 0; w < kDmaThreads / 64; w++) base += w < wave ? us.part[w] : 0;
        const int first = base + incl - nr;
        if (tid < nrows && first <= g && g < first + nr) {
            const int k = g - first, q_u = u / nr, r_u = u % nr;
            us.run[0] = tid;
            us.run[1] = k * q_u + (k < r_u ? k : r_u);
            us.run[2] = q_u + (k < r_u ? 1 : 0);
            us.run[3] = k == nr - 1;
            us.run_len = Lr;
        }
        if (tid == nrows - 1) us.run[4] = first + nr;
        __syncthreads();
    }
    if (g >= us.run[4]) return;                        // more blocks than runs
    const int row = __builtin_amdgcn_readfirstlane(us.run[0]);
    const int64_t blk0 = (int64_t)kUnitKeys * __builtin_amdgcn_readfirstlane(us.run[1]);
    const int64_t span = (int64_t)kUnitKeys * __builtin_amdgcn_readfirstlane(us.run[2]);
    const bool last_run = __builtin_amdgcn_readfirstlane(us.run[3]) != 0;
    const int64_t Lrow = us.run_len;
    // ---- the run: row `row`, keys [blk0, blk0 + span)
    const int qrow = row;
    const int b = row;
    const int64_t T = a.rows.T;
    const int64_t L = Lrow;
    float *out = a.scores + (int64_t)qrow * T;
    const int64_t end = last_run ? T : blk0 + span;    // the slots this block answers for
    const bool loader = wave >= kDmaComputeWaves;
    const int head = tid >> 3, sub = tid & 7;
    const bool rope_on = a.rope_cos != nullptr;
    if (blk0 >= L) {                                   // an empty row: -inf (and its quantized query)
        if (loader) return;
        for (int64_t s = blk0 + tid; s < end && s < T; s += 64 * kDmaComputeWaves) out[s] = -__builtin_inff();
        if (kFused && blk0 == 0 && a.q_fp8_out) {
            const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_bf16 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
            const uint4 q0 = qs[0], q1 = qs[1];
            uint32_t in[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            if (rope_on) {
                Rope16 rr;
                load_rope16(a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2), a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2), sub, rr);
                rope_row16(in, rr, sub);
            }
            uint32_t codes[4];
            int j;
            quantize_row16(in, codes, j);
            *reinterpret_cast<uint4 *>(a.q_fp8_out + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub) =
                make_uint4(codes[0], codes[1], codes[2], codes[3]);
            if (sub == 0) a.w_eff_out[(int64_t)qrow * LK_HEADS + head] = fold_weight(a.w[(int64_t)qrow * LK_HEADS + head], j);
        }
        return;
    }
    const uint8_t *kbase = a.k_cache + (int64_t)b * a.cache_seq_stride * LK_DIM;
    // units holding a valid key (uniform, >= 1 here); the slots past them are only -inf
    const int nunits = (int)((L - blk0 < span ? L - blk0 + kUnitKeys - 1 : span) / kUnitKeys);
    const int NP = kUnitTiles * nunits;                // phases: one tile of every compute wave each
    if (loader) {
        // Loader wave v: in phase P (tile P % 2 of unit P / 2), DMA instruction i covers
        // phase rows 8 (v * kDmaPerPhase + i) .. +7; phase P lands in buffer P % 4.
        const int v = wave - kDmaComputeWaves;
        auto issue_phase = [&](int P) {
            const int p = P & (kUnitTiles - 1);
            const int64_t ub = blk0 + (int64_t)kUnitKeys * (P / kUnitTiles);
            uint8_t *buf = sm.k + (P & (kDecTiles - 1)) * kDmaPhaseBytes;
#pragma unroll
            for (int i = 0; i < kDmaPerPhase; i++) {
                const int R = 8 * (v * kDmaPerPhase + i) + (lane >> 3);   // row within the phase
                const int w = R >> 5, r = R & 31;
                const int q = kslot(r, lane & 7);                         // the chunk this lane's slot holds
                const int64_t s = ub + 64 * w + 32 * p + r;
                const uint8_t *src = kbase + (s < L ? s : 0) * LK_DIM + 16 * q;
                dma_b128(src, buf + 1024 * (v * kDmaPerPhase + i));
            }
        };
        issue_phase(0);
        issue_phase(1);                                // NP >= 2
#pragma unroll 1
        for (int P = 0; P < NP; P++) {                 // one barrier per phase, as the compute waves
            if (P + 1 < NP) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerPhase));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();                           // phase P landed (P = 0: and the query is prepared)
            if (P + 2 < NP) issue_phase(P + 2);        // into the buffer of phase P - 2, read before barrier P
        }
        return;
    }

    // Compute wave `wave`: in unit j, keys blk0 + 512 j + 64 wave .. + 63 (tile p: + 32 p).
    int64_t pn = -1;                                   // the new key's slot (uniform; none unfused)
    const float *sbase = a.k_scale + (int64_t)b * a.cache_seq_stride;
    float ks_u;                                        // key scale of this lane's key in the current unit
    if constexpr (kFused) {
        pn = L - 1 < blk0 + span ? L - 1 : -1;
        const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_bf16 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
        const uint4 qp0 = qs[0], qp1 = qs[1];
        const float wr = a.w[(int64_t)qrow * LK_HEADS + head];
        const uint32_t kn = reinterpret_cast<const uint32_t *>(a.k_new + (int64_t)b * LK_DIM)[lane];
        const float *kc_row = rope_on ? a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2) : reinterpret_cast<const float *>(a.k_new);
        const float *ks_row = rope_on ? a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2) : reinterpret_cast<const float *>(a.k_new);
        const float2 krc = reinterpret_cast<const float2 *>(kc_row)[lane & 15];
        const float2 krs = reinterpret_cast<const float2 *>(ks_row)[lane & 15];
        Rope32 rope_row;
        if (rope_on)
            load_rope32_uniform(a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2),
                                a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2), rope_row);
        {
            const int64_t s = blk0 + 64 * wave + lane;
            ks_u = sbase[s < L ? s : 0];
        }
        {
            uint32_t in[8] = {qp0.x, qp0.y, qp0.z, qp0.w, qp1.x, qp1.y, qp1.z, qp1.w};
            if (rope_on) {
                Rope16 rope;
                pick_rope16(rope_row, sub, rope);
                rope_row16(in, rope, sub);
            }
            uint32_t codes[4];
            int j;
            quantize_row16(in, codes, j);
            const uint4 piece = make_uint4(codes[0], codes[1], codes[2], codes[3]);
            *reinterpret_cast<uint4 *>(sq + head * kQPitch + 16 * sub) = piece;
            const float we = fold_weight(wr, j);
            if (sub == 0) sw[head] = we;
            if (blk0 == 0 && a.q_fp8_out) {
                *reinterpret_cast<uint4 *>(a.q_fp8_out + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub) = piece;
                if (sub == 0) a.w_eff_out[(int64_t)qrow * LK_HEADS + head] = we;
            }
        }
        if (pn >= 0 && wave == 0) {                        // the new key, spread over wave 0 (2 features a lane)
            uint32_t kin = kn;
            if (rope_on) rope_row_wave(kin, krc, krs);
            int kj;
            const uint32_t kc = quantize_row_wave(kin, kj);
            const int64_t row_off = (int64_t)b * a.cache_seq_stride + pn;
            reinterpret_cast<uint16_t *>(a.k_cache + row_off * LK_DIM)[lane] = (uint16_t)kc;
            reinterpret_cast<uint16_t *>(snew)[lane] = (uint16_t)kc;
            if (lane == 0) {
                const float ksc = __builtin_ldexpf(1.0f, kj);
                a.k_scale[row_off] = ksc;
                sm.d.snew_scale = ksc;
            }
        }
    } else {                                           // lk_index_score: the prepared query
        const uint4 piece =
            *reinterpret_cast<const uint4 *>(a.q_fp8 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
        const float we = a.w_eff[(int64_t)qrow * LK_HEADS + head];
        const int64_t s = blk0 + 64 * wave + lane;
        ks_u = sbase[s < L ? s : 0];
        *reinterpret_cast<uint4 *>(sq + head * kQPitch + 16 * sub) = piece;
        if (sub == 0) sw[head] = we;
    }
    __syncthreads();                                   // query prepared, phase 0 landed
    QueryRaw raw;
    {
        const int r = lane & 31, hh = lane >> 5;
#pragma unroll
        for (int m = 0; m < 2; m++) {
            const uint8_t *qr = sq + (32 * m + r) * kQPitch + 64 * hh;
#pragma unroll
            for (int c = 0; c < 4; c++) raw.q[m][c] = *reinterpret_cast<const uint4 *>(qr + 16 * c);
#pragma unroll
            for (int gq = 0; gq < 4; gq++) raw.w[m][gq] = *reinterpret_cast<const float4 *>(sw + 32 * m + 8 * gq + 4 * hh);
        }
    }
    QueryFrag f;
    convert_query(raw, f);
    // The lane-derived LDS addresses are recomputed where they are used: held across the
    // unit loop they would not fit the register budget.
    auto opaque_lane = [&]() {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        return ln;
    };
    // relu_weighted_sum with the weights read from LDS two quads at a time, in its order.
    auto relu_weighted_sum_lds = [&](const float16v (&acc2)[2]) {
        const int hh = opaque_lane() >> 5;
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i0 = 0; i0 < 8; i0 += 2) {
            float4 wq[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = (i0 + i) >> 2, gq = (i0 + i) & 3;
                wq[i] = *reinterpret_cast<const float4 *>(sw + 32 * m + 8 * gq + 4 * hh);
            }
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = (i0 + i) >> 2, gq = (i0 + i) & 3;
                const float wg[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
#pragma unroll
                for (int kk = 0; kk < 4; kk++)
                    s4[kk] = __builtin_fmaf(__builtin_fmaxf(acc2[m][4 * gq + kk], 0.0f), wg[kk], s4[kk]);
            }
        }
        return (s4[0] + s4[1]) + (s4[2] + s4[3]);
    };
    // Phase P's tile of this wave: its 32 keys from buffer P % 4 through the MFMAs.
    auto tile = [&](int P, int64_t kj, int p, float16v (&accd)[2]) {
        const int ln = opaque_lane();
        const int r = ln & 31, hh = ln >> 5;
        uint4 kv[4];
        const uint8_t *rowp = sm.k + (P & (kDecTiles - 1)) * kDmaPhaseBytes + (32 * wave + r) * LK_DIM;
#pragma unroll
        for (int c = 0; c < 4; c++) kv[c] = *reinterpret_cast<const uint4 *>(rowp + 16 * kslot(r, 4 * hh + c));
        const bool mine = kj + 32 * p + r == pn;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const uint4 n = snew[4 * hh + c];
            kv[c].x = mine ? n.x : kv[c].x;
            kv[c].y = mine ? n.y : kv[c].y;
            kv[c].z = mine ? n.z : kv[c].z;
            kv[c].w = mine ? n.w : kv[c].w;
        }
        mfma_tile(kv, f, accd);
    };
    const float nscale = sm.d.snew_scale;
    float16v acc[2][2];
#pragma unroll 1
    for (int j = 0; j < nunits; j++) {
        const int64_t kj = blk0 + (int64_t)kUnitKeys * j + 64 * wave;
        if (j > 0) __syncthreads();                    // phase 2 j landed
        tile(2 * j, kj, 0, acc[0]);
        float ks_next = 0.0f;
        if (j + 1 < nunits) {                          // the next unit's key scale
            const int64_t s = kj + kUnitKeys + lane;
            ks_next = sbase[s < L ? s : 0];
        }
        __syncthreads();                               // phase 2 j + 1 landed
        tile(2 * j + 1, kj, 1, acc[1]);
        const float p0 = relu_weighted_sum_lds(acc[0]);
        const float sum = halves_sum_pair(p0, relu_weighted_sum_lds(acc[1]));
        const int64_t s = kj + lane;                   // lanes 0-31: tile 0's keys, 32-63: tile 1's
        const float ksv = s == pn ? nscale : ks_u;
        const float v = s < L ? sum * ksv : -__builtin_inff();
        if (s < T) out[s] = v;
        ks_u = ks_next;
    }
    for (int64_t s = blk0 + (int64_t)kUnitKeys * nunits + tid; s < end && s < T; s += 64 * kDmaComputeWaves)
        out[s] = -__builtin_inff();
}

// ------------------------------------------------------------------ decode, standalone score
// lk_index_score with S == 1 and a prepared query: one block per (row, 1024-key block),
// four waves (one per SIMD), each scoring 256 consecutive keys as 8 tiles through
// pipelined_tiles with kPipeFly tiles in flight.  Without a preparation to cover, fewer
// and longer waves stream K best: the query staging is short, and a single wave per
// SIMD keeps its tiles' loads ahead of its MFMAs.
constexpr int kPipeWaves = 4;
constexpr int kPipeThreads = 64 * kPipeWaves;
constexpr int kPipeTiles = 8;
constexpr int kPipeFly = 4;
static_assert(kPipeWaves * kPipeTiles * 32 == kDecKeysPerBlock, "1024-key blocks, as the other decode kernels");
static_assert(LK_HEADS * LK_DIM / 16 == 2 * kPipeThreads, "two 16-byte query pieces per thread");

__global__ void __launch_bounds__(kPipeThreads) decode_pipe_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sq[LK_HEADS * kQPitch];
    __shared__ __attribute__((aligned(16))) float sw[LK_HEADS];
    LK_POISON_LDS_OBJS(sq, sw);
    const int qrow = blockIdx.y;
    const int64_t blk0 = (int64_t)blockIdx.x * kDecKeysPerBlock;
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
    const int b = qrow / a.rows.S;
    const int t = qrow - b * a.rows.S;
    const int64_t T = a.rows.T;
    const int64_t L = row_len(a.rows, b, t);
    const int64_t key0 = blk0 + (int64_t)wave * (32 * kPipeTiles);
    float *out = a.scores + (int64_t)qrow * T;
    if (blk0 >= L) {                                   // the whole block is masked: -inf only
        for (int64_t s = blk0 + threadIdx.x; s < blk0 + kDecKeysPerBlock && s < T; s += kPipeThreads)
            out[s] = -__builtin_inff();
        return;
    }
    const int r = lane & 31, hh = lane >> 5;
    // Query pieces tid and tid + 256 (head piece / 8, 16-byte chunk piece % 8) and a
    // float4 of the weights, issued before the K loads.
    const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_fp8 + (int64_t)qrow * LK_HEADS * LK_DIM);
    const uint4 qf0 = qs[threadIdx.x], qf1 = qs[threadIdx.x + kPipeThreads];
    const float4 wv = reinterpret_cast<const float4 *>(a.w_eff + (int64_t)qrow * LK_HEADS)[lane & 15];
    float ks[kPipeTiles / 2];
#pragma unroll
    for (int p = 0; p < kPipeTiles / 2; p++) {
        const int64_t s = key0 + 64 * p + lane;
        ks[p] = a.k_scale[(int64_t)b * a.cache_seq_stride + (s < L ? s : 0)];
    }
    const uint8_t *kbase = a.k_cache + (int64_t)b * a.cache_seq_stride * LK_DIM;
    uint4 kv[kPipeTiles][4];
    auto load_tile = [&](int j) {
        const int64_t s = key0 + 32 * j + r;
        const uint4 *src = reinterpret_cast<const uint4 *>(kbase + (s < L ? s : 0) * LK_DIM + 64 * hh);
#pragma unroll
        for (int c = 0; c < 4; c++) kv[j][c] = src[c];       // rows past L re-read row 0 (masked below)
    };
#pragma unroll
    for (int j = 0; j < kPipeFly; j++) load_tile(j);
    __builtin_amdgcn_sched_barrier(0);
    const int piece = threadIdx.x;
    *reinterpret_cast<uint4 *>(sq + (piece >> 3) * kQPitch + 16 * (piece & 7)) = qf0;
    *reinterpret_cast<uint4 *>(sq + ((piece + kPipeThreads) >> 3) * kQPitch + 16 * (piece & 7)) = qf1;
    reinterpret_cast<float4 *>(sw)[lane & 15] = wv;    // duplicate stores of equal values
    __syncthreads();
    QueryRaw raw;
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const uint8_t *qr = sq + (32 * m + r) * kQPitch + 64 * hh;
#pragma unroll
        for (int c = 0; c < 4; c++) raw.q[m][c] = *reinterpret_cast<const uint4 *>(qr + 16 * c);
#pragma unroll
        for (int g = 0; g < 4; g++) raw.w[m][g] = *reinterpret_cast<const float4 *>(sw + 32 * m + 8 * g + 4 * hh);
    }
    QueryFrag f;
    convert_query(raw, f);
    pipelined_tiles<kPipeTiles, kPipeFly>(kv, load_tile, f, ks, key0, T, L, out);
}

// ------------------------------------------------------------------ prefill (S > 1)
// A block of 8 waves (two per SIMD) owns 8 consecutive query tokens of one sequence (one
// per wave) and a slice of keys (the group's whole key range when the token groups fill
// the chip, else up to 4096 keys), taken as chunks of 256.  Each chunk is read
// from HBM once per block, converted to f16 once and kept in LDS (two 68 KB buffers),
// where every wave streams it through the MFMA against its own query held in registers;
// the chunks are double buffered, so one barrier per chunk (eight tiles per wave)
// publishes the next one.
//  - Staging layout: thread (wave w, lane l) stages key row 32 w + l % 32 of the chunk,
//    half l / 32 of the row, and writes it to LDS in the MFMA B-operand read pattern
//    (rows in lanes 0-31, the other half of the row in lanes 32-63): the pattern in
//    which the 16-byte LDS accesses are free of bank conflicts.
//  - The next chunk's loads are issued at the start of a chunk; their conversion and LDS
//    writes ride in the MFMA stream of the chunk's third tile.
//  - Chunks valid for the wave's row run as one software pipeline across chunk
//    boundaries: step g issues the 16 MFMAs of tile g, then the ReLU / weight / head-sum
//    epilogue of tile g - 1 (two tiles make 64 keys, one per lane after a cross-half
//    swap), so the VALU epilogue runs in the shadow of the matrix core.  The chunk that
//    holds the row's last valid key runs the same pipeline over its tile pairs up to
//    that key, with the stores masked; later chunks of the row are only written -inf.
//  - Work items (sequence, token group, slice) are numbered slice fastest and token
//    groups from the last (longest causal rows first); the 1-D grid is dispatched to the
//    8 XCDs round-robin, so block 8p + x (XCD x) takes item 8p + (x + p) % 8, which
//    gives every XCD every slice equally often instead of pinning slice x to XCD x.
constexpr int kPreWaves = 8;                          // query tokens per block, one per wave
constexpr int kPreThreads = 64 * kPreWaves;
constexpr int kPreChunk = 256;                        // keys per LDS buffer
constexpr int kPreTiles = kPreChunk / 32;
constexpr int kPreChunks = 16;                        // chunks per slice when rows are split
constexpr int kPreSlice = kPreChunk * kPreChunks;     // keys per work item when rows are split
constexpr int kPreRowBytes = 2 * LK_DIM + 16;         // f16 row + 16 B pad against bank conflicts
constexpr int kPreRowGroups = kPreChunk / 32;         // 32-row groups of a chunk
constexpr int kPrePieces = 2 * kPreWaves / kPreRowGroups;   // pieces each key row is staged in
constexpr int kPrePieceBytes = LK_DIM / kPrePieces;         // fp8 bytes staged per thread
constexpr int kPreStageTile = 2;                      // tile whose MFMA stream carries the staging
static_assert(kPreRowGroups <= kPreWaves && kPrePieces * kPrePieceBytes == LK_DIM && kPrePieceBytes % 16 == 0,
              "staging map");
static_assert(kPreChunk <= kPreThreads, "one key scale per thread");
static_assert(kPreTiles % 2 == 0 && kPreStageTile < kPreTiles, "tile pairs never straddle a chunk");

// One thread's share of a chunk in flight: kPrePieceBytes of one key row and, for
// threads below kPreChunk, one key scale.
struct ChunkPart {
    uint4 v[kPrePieceBytes / 16];
    float ks;
};

__device__ __forceinline__ int stage_row() { return 32 * ((threadIdx.x >> 6) % kPreRowGroups) + (threadIdx.x & 31); }
__device__ __forceinline__ int stage_piece() {
    return ((threadIdx.x >> 5) & 1) + 2 * ((threadIdx.x >> 6) / kPreRowGroups);
}

// Rows at or past Lmax (no row of the block needs them) re-read row 0 and are never used.
__device__ __forceinline__ void load_chunk_part(const uint8_t *__restrict__ kbase, const float *__restrict__ sbase,
                                                int64_t kc, int64_t Lmax, ChunkPart &p) {
    const int64_t s = kc + stage_row();
    const uint4 *src = reinterpret_cast<const uint4 *>(kbase + (s < Lmax ? s : 0) * LK_DIM +
                                                       kPrePieceBytes * stage_piece());
#pragma unroll
    for (int c = 0; c < kPrePieceBytes / 16; c++) p.v[c] = src[c];
    p.ks = (threadIdx.x < kPreChunk && kc + threadIdx.x < Lmax) ? sbase[kc + threadIdx.x] : 0.0f;
}

__device__ __forceinline__ void store_chunk_part(uint8_t *sk, float *sks, const ChunkPart &p) {
    half8 *dst = reinterpret_cast<half8 *>(sk + stage_row() * kPreRowBytes + 2 * kPrePieceBytes * stage_piece());
#pragma unroll
    for (int c = 0; c < kPrePieceBytes / 16; c++) {
        dst[2 * c] = fp8x8_to_half8(p.v[c].x, p.v[c].y);
        dst[2 * c + 1] = fp8x8_to_half8(p.v[c].z, p.v[c].w);
    }
    if (threadIdx.x < kPreChunk) sks[threadIdx.x] = p.ks;
}

int cu_count();

// Work items of the prefill grid (see above).  When the token groups alone give every
// compute unit at least two blocks, a block takes its group's whole key range (one
// slice), so the query load, the first chunk's staging and the pipeline fill happen
// once per group; otherwise rows are split into slices of kPreSlice keys.
struct PrefillGrid {
    int nslices, nrg, n_items;
    int slice_chunks;                                 // chunks per slice
    int64_t slice_keys;                               // slice_chunks * kPreChunk
};
PrefillGrid prefill_grid(const RowsDev &rows) {
    PrefillGrid g;
    g.nrg = (rows.S + kPreWaves - 1) / kPreWaves;
    const int64_t tchunks = (rows.T + kPreChunk - 1) / kPreChunk;
    const int64_t groups = (int64_t)rows.B * g.nrg;
    int64_t sc = kPreChunks;
    if (groups >= 2 * (int64_t)cu_count() && tchunks > sc && tchunks <= (1 << 24)) sc = tchunks;
    g.slice_chunks = (int)sc;
    g.slice_keys = sc * kPreChunk;
    g.nslices = (int)((rows.T + g.slice_keys - 1) / g.slice_keys);
    g.n_items = g.nslices * g.nrg * rows.B;
    return g;
}

__global__ void __launch_bounds__(kPreThreads)
score_prefill_kernel(const uint8_t *__restrict__ q_fp8, const float *__restrict__ w_eff,
                     const uint8_t *__restrict__ k_cache, const float *__restrict__ k_scale,
                     int64_t cache_seq_stride, RowsDev rows, float *__restrict__ scores, PrefillGrid grid) {
    __shared__ __attribute__((aligned(16))) uint8_t sk[2][kPreChunk * kPreRowBytes];
    __shared__ float sks[2][kPreChunk];
    LK_POISON_LDS_OBJS(sk, sks);
    const int p8 = (int)(blockIdx.x >> 3), x8 = (int)(blockIdx.x & 7);
    const int item = (p8 << 3) + ((x8 + p8) & 7);
    if (item >= grid.n_items) return;
    const int slice = item % grid.nslices;
    const int rg = grid.nrg - 1 - (item / grid.nslices) % grid.nrg;
    const int b = item / (grid.nslices * grid.nrg);
    const int lane = __lane_id();
    const int wave = threadIdx.x >> 6;
    const int t0 = rg * kPreWaves;
    const int64_t T = rows.T;
    const int64_t slice0 = (int64_t)slice * grid.slice_keys;
    const int t = t0 + wave;
    const bool has_row = t < rows.S;
    const int64_t L = has_row ? row_len(rows, b, t) : 0;
    // The block needs keys below the largest valid length of its rows.
    const int t_last = (t0 + kPreWaves - 1 < rows.S ? t0 + kPreWaves - 1 : rows.S - 1);
    const int64_t Lmax = row_len(rows, b, t_last);     // row_len is non-decreasing in t
    float *out = scores + ((int64_t)b * rows.S + t) * T;
    // Chunks of the slice with any valid key for some row of the block.
    const int64_t live = Lmax - slice0;
    const int nchunks = live <= 0 ? 0
                      : (live >= grid.slice_keys ? grid.slice_chunks : (int)((live + kPreChunk - 1) / kPreChunk));
    // -inf for this row's slots of the chunks no row of the block needs.
    if (has_row)
        for (int64_t s = slice0 + (int64_t)nchunks * kPreChunk + lane; s < slice0 + grid.slice_keys && s < T; s += 64)
            out[s] = -__builtin_inff();
    if (nchunks == 0) return;
    // Chunks in which every key is valid for this row: [0, nfull).
    const int64_t lrow = L - slice0;
    const int nfull = lrow <= 0 ? 0 : (lrow >= (int64_t)nchunks * kPreChunk ? nchunks : (int)(lrow / kPreChunk));

    const uint8_t *kbase = k_cache + (int64_t)b * cache_seq_stride * LK_DIM;
    const float *sbase = k_scale + (int64_t)b * cache_seq_stride;
    ChunkPart part;
    load_chunk_part(kbase, sbase, slice0, Lmax, part);
    QueryFrag f;
    if (has_row) {
        const int64_t qrow = (int64_t)b * rows.S + t;
        load_query(q_fp8 + qrow * LK_HEADS * LK_DIM, w_eff + qrow * LK_HEADS, lane, f);
    }
    store_chunk_part(sk[0], sks[0], part);
    __syncthreads();
    const int r = lane & 31, hh = lane >> 5;
    auto mfma_tile = [&](const uint8_t *skc, int j, float16v acc[2]) {
        const uint8_t *rowbase = skc + (32 * j + r) * kPreRowBytes + 128 * hh;
        acc[0] = float16v{};
        acc[1] = float16v{};
#pragma unroll
        for (int kk = 0; kk < 8; kk++) {
            const half8 bk = *reinterpret_cast<const half8 *>(rowbase + 16 * kk);
#pragma unroll
            for (int m = 0; m < 2; m++)
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[m][kk], bk, acc[m], 0, 0, 0);
        }
    };
    // The pipeline over the valid chunks.  Tiles 2i and 2i + 1 of a chunk make 64 keys
    // (lanes 0-31 and 32-63 after halves_sum_pair); the key scales of a pair are read
    // into a register right after the previous pair's store.  The chunk in which the
    // row's valid prefix ends runs the same pipeline over its tile pairs up to the one
    // holding key L - 1 (jmax tiles), with the stores masked past L and T.
    float16v acc[2][2];
    float p0 = 0.f, ks_pair = 0.f;
    int64_t s_pair = 0;
    bool owed = false;                                 // a computed tile still owes its epilogue
    auto store_pair = [&](float v, auto masked) {
        const int64_t s = s_pair + lane;
        if constexpr (decltype(masked)::value) {
            if (s < T) out[s] = s < L ? v * ks_pair : -__builtin_inff();
        } else {
            out[s] = v * ks_pair;                      // s < L <= T
        }
    };
    auto run_chunk = [&](int c, int jmax, auto masked) {
        const int64_t kc = slice0 + (int64_t)c * kPreChunk;
        const bool more = c + 1 < nchunks;
        if (more) load_chunk_part(kbase, sbase, kc + kPreChunk, Lmax, part);   // in flight during the MFMA work
        const uint8_t *skc = sk[c & 1];
        const float *sksc = sks[c & 1];
#pragma unroll
        for (int j = 0; j < kPreTiles; j++) {
            __builtin_amdgcn_sched_barrier(0);
            if (decltype(masked)::value && j >= jmax) {   // past the row's last tile pair
                if (j == kPreStageTile && more) store_chunk_part(sk[(c + 1) & 1], sks[(c + 1) & 1], part);
                continue;
            }
            mfma_tile(skc, j, acc[j & 1]);
            if (owed) {                                // the epilogue of the previous tile
                const float pv = relu_weighted_sum(acc[(j + 1) & 1], f);
                if (j & 1) p0 = pv;                    // the previous tile is the first of a pair
                else store_pair(halves_sum_pair(p0, pv), masked);
            }
            if ((j & 1) == 0) {
                ks_pair = sksc[32 * j + lane];
                s_pair = kc + 32 * j;
            }
            owed = true;
            // One scheduling region per step: the tile's 8 operand reads first, then part
            // of the epilogue while they land, then the MFMA chain interleaved with the
            // rest of the epilogue (and, in the staging tile, the next chunk's LDS writes).
            if (j == kPreStageTile) {
                if (more) store_chunk_part(sk[(c + 1) & 1], sks[(c + 1) & 1], part);
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);       // DS reads
                __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);      // VALU
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    for (int c = 0; c < nfull; c++) run_chunk(c, kPreTiles, std::false_type{});
    // The chunk holding key L - 1, if it is not a full one: its valid tile pairs.
    int c2 = nfull;
    if (has_row && nfull < nchunks && lrow > (int64_t)nfull * kPreChunk) {
        const int64_t kc = slice0 + (int64_t)nfull * kPreChunk;
        const int np = (int)((L - kc + 63) / 64);      // 1 .. kPreTiles / 2
        run_chunk(nfull, 2 * np, std::true_type{});
        const float pv = relu_weighted_sum(acc[1], f);  // its last tile (2 np - 1 is odd)
        store_pair(halves_sum_pair(p0, pv), std::true_type{});
        owed = false;
        for (int64_t s = kc + 64 * np + lane; s < kc + kPreChunk && s < T; s += 64) out[s] = -__builtin_inff();
        c2 = nfull + 1;
    }
    if (owed) {                                        // the last valid chunk's last tile
        const float pv = relu_weighted_sum(acc[(kPreTiles - 1) & 1], f);
        store_pair(halves_sum_pair(p0, pv), std::false_type{});
    }
    // Chunks past the one holding key L - 1 (every chunk, for rows past S): no valid key
    // for this row.  The wave writes them -inf, stages its share of the next chunk and
    // passes the chunk's barrier, so every wave passes one barrier per chunk.
    for (int c = c2; c < nchunks; c++) {
        const int64_t kc = slice0 + (int64_t)c * kPreChunk;
        const bool more = c + 1 < nchunks;
        if (more) load_chunk_part(kbase, sbase, kc + kPreChunk, Lmax, part);
        if (has_row)
            for (int64_t s = kc + lane; s < kc + kPreChunk && s < T; s += 64) out[s] = -__builtin_inff();
        if (more) store_chunk_part(sk[(c + 1) & 1], sks[(c + 1) & 1], part);
        __syncthreads();
    }
}

// Compute units of the current device (queried once per device).
int cu_count() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Decode grid (S == 1): one block per (row, key block) when that fits the chip about
// once; beyond, balanced runs of 512-key units, one block per compute unit (or per row
// when the rows outnumber them).
template <bool kFused>
hipError_t launch_decode_grid(const DecodeArgs &a, hipStream_t stream) {
    const RowsDev &rows = a.rows;
    const int64_t nblk = (rows.T + kDecKeysPerBlock - 1) / kDecKeysPerBlock;
    const int64_t nrows = (int64_t)rows.B * rows.S;
    const int cus = cu_count();
    if (nrows <= kUnitMaxRows && nblk * nrows * 4 > (int64_t)cus * 5) {
        const unsigned grid = (unsigned)(nrows > cus ? nrows : cus);   // S == 1: runs of 512-key units
        return launch(decode_units_kernel<kFused>, dim3(grid), dim3(kDmaThreads), 0u, stream, a);
    }
    dim3 grid((unsigned)nblk, (unsigned)rows.B);
    if constexpr (kFused) return launch(decode_kernel<false>, grid, dim3(kDmaThreads), 0u, stream, a);
    return launch(decode_pipe_kernel, grid, dim3(kPipeThreads), 0u, stream, a);
}

}  // namespace

// Whether lk_index_score's grid for these rows is within the launch limits.
bool index_score_grid_fits(const RowsDev &rows) {
    if (rows.B > 65535) return false;
    if (rows.S == 1) return (rows.T + kDecKeysPerBlock - 1) / kDecKeysPerBlock <= 0x7FFFFFFF;
    // prefill: one block per (sequence, 8-token group, 4096-key slice), rounded up to 8
    const int64_t items = (int64_t)rows.B * ((rows.S + kPreWaves - 1) / kPreWaves) *
                          ((rows.T + kPreSlice - 1) / kPreSlice);
    return (items + 7) / 8 * 8 <= 0x7FFFFFFF;
}

hipError_t launch_index_score(const uint8_t *q_fp8, const float *w_eff, const uint8_t *k_cache,
                              const float *k_scale, int64_t cache_seq_stride, const RowsDev &rows,
                              float *scores, hipStream_t stream) {
    if (rows.S == 1) {
        DecodeArgs a{};
        a.q_fp8 = q_fp8;
        a.w_eff = w_eff;
        a.k_cache = const_cast<uint8_t *>(k_cache);    // read only: the standalone kernel never writes it
        a.k_scale = const_cast<float *>(k_scale);
        a.cache_seq_stride = cache_seq_stride;
        a.rows = rows;
        a.scores = scores;
        return launch_decode_grid<false>(a, stream);
    } else {
        const PrefillGrid g = prefill_grid(rows);
        const unsigned blocks = (unsigned)((g.n_items + 7) / 8 * 8);
        return launch(score_prefill_kernel, dim3(blocks), dim3(kPreThreads), 0u, stream, q_fp8, w_eff, k_cache,
                      k_scale, cache_seq_stride, rows, scores, g);
    }
}

// The fused decode step: S == 1 rows, query quantization and the new key's write
// done inside the score kernel.
hipError_t launch_decode_score(const uint16_t *q, const float *w, const uint16_t *k_new, uint8_t *k_cache,
                               float *k_scale, int64_t cache_seq_stride, const RowsDev &rows, float *scores,
                               uint8_t *q_fp8_out, float *w_eff_out, const float *rope_cos,
                               const float *rope_sin, hipStream_t stream) {
    DecodeArgs a{};
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.q_bf16 = q;
    a.w = w;
    a.k_new = k_new;
    a.q_fp8_out = q_fp8_out;
    a.w_eff_out = w_eff_out;
    a.k_cache = k_cache;
    a.k_scale = k_scale;
    a.cache_seq_stride = cache_seq_stride;
    a.rows = rows;
    a.scores = scores;
    return launch_decode_grid<true>(a, stream);
}

hipError_t launch_topk(const float *scores, const RowsDev &rows, int32_t k, int32_t *idx, hipStream_t stream);

// The fused decode step with its top-k: rows of at most one key block in one launch
// (decode_kernel<true>: scores kept in LDS, the top-k by the block's loader waves);
// longer rows as the fused score launch followed by the top-k launch (scores required).
hipError_t launch_decode_select(const uint16_t *q, const float *w, const uint16_t *k_new, uint8_t *k_cache,
                                float *k_scale, int64_t cache_seq_stride, const RowsDev &rows, float *scores,
                                uint8_t *q_fp8_out, float *w_eff_out, const float *rope_cos,
                                const float *rope_sin, int32_t k, int32_t *idx, hipStream_t stream) {
    if (rows.T > kDecKeysPerBlock) {
        const hipError_t e = launch_decode_score(q, w, k_new, k_cache, k_scale, cache_seq_stride, rows, scores,
                                                 q_fp8_out, w_eff_out, rope_cos, rope_sin, stream);
        return e != hipSuccess ? e : launch_topk(scores, rows, k, idx, stream);
    }
    DecodeArgs a{};
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.q_bf16 = q;
    a.w = w;
    a.k_new = k_new;
    a.q_fp8_out = q_fp8_out;
    a.w_eff_out = w_eff_out;
    a.k_cache = k_cache;
    a.k_scale = k_scale;
    a.cache_seq_stride = cache_seq_stride;
    a.rows = rows;
    a.scores = scores;
    a.k = k;
    a.idx = idx;
    return launch(decode_kernel<true>, dim3(1, (unsigned)rows.B), dim3(kDmaThreads), 0u, stream, a);
}

}  // namespace lk

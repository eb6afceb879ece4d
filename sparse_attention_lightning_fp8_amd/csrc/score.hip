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
#include "lk_device.h"
#include "quant_device.h"

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

// Scores of one 32-key tile whose B operand (this lane's 64 bytes of key l % 32) is `kv`.
__device__ __forceinline__ float score_tile(const uint4 kv[4], const QueryFrag &f) {
    float16v acc[2] = {};
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
    return relu_weighted_sum(acc, f);
}

// ------------------------------------------------------------------ decode (S == 1)
// One wave scores 128 consecutive keys (4 tiles of 32) of one query row; a block of
// kDecWaves waves covers kDecKeysPerBlock keys of that row.  Each lane loads its
// 4 x 64 bytes of K straight into the B-operand registers (keys are read exactly
// once, so staging K in LDS brings no reuse).  The query (8 KB as e4m3fn) and its
// weights (256 B) are needed by every wave: the block fetches them once into LDS and
// each wave takes its A fragments from there.
// Order of work: the query loads, then every K load of the wave (16 KB in flight),
// then the query staging while K streams in, then the tiles in arrival order.
//
// The fused variant (lk_decode_score) starts from the bf16 query, the raw weights
// and the new key of the decode step: each block quantizes the row's 64 query heads
// itself (8 lanes per head, the same arithmetic as lk_quantize_queries) while its K
// loads are in flight, and the block holding key L-1 (the new token's slot) also
// rotates and quantizes the new key, writes it to the cache, and hands it to the
// lanes that score it in place of the stale cache row they loaded.
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
    float *scores;              // [B, T]
};

struct DecodeShared {
    uint8_t sq[LK_HEADS * kQPitch];             // the row's quantized query (A operand source)
    float sw[LK_HEADS];                         // its folded weights
    uint4 snew[8];                              // fused: the new key's 128 codes
    float snew_scale;
};

// Keys [blk0, blk0 + kDecKeysPerBlock) of score row qrow (one block's work item).
// prep: bring in (fused: quantize) the row's query; otherwise sq and sw already hold
// this row's query from the block's previous item.  `first`: the block's first item (a
// later item that rewrites sq waits for every wave to be done with it).
template <bool kFused, bool prep>
__device__ __forceinline__ void decode_item(const DecodeArgs &a, DecodeShared &sm, int qrow, int64_t blk0,
                                            bool first) {
    uint8_t *const sq = sm.sq;
    float *const sw = sm.sw;
    uint4 *const snew = sm.snew;
    const int lane = __lane_id();
    const int wave = threadIdx.x >> 6;
    const int b = qrow / a.rows.S;
    const int t = qrow - b * a.rows.S;
    const int64_t T = a.rows.T;
    const int64_t L = row_len(a.rows, b, t);
    const int64_t key0 = blk0 + (int64_t)wave * kDecKeysPerWave;
    float *out = a.scores + (int64_t)qrow * T;
    const int head = threadIdx.x >> 3, sub = threadIdx.x & 7;   // fused: this thread's 16 features of a head
    if (blk0 >= L) {                                   // the whole block is masked: -inf only
        for (int64_t s = blk0 + threadIdx.x; s < blk0 + kDecKeysPerBlock && s < T; s += kDecThreads)
            out[s] = -__builtin_inff();
        if constexpr (kFused) {                        // a row with L == 0 still returns its quantized query
            if (blk0 == 0 && a.q_fp8_out) {
                const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_bf16 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
                const uint4 q0 = qs[0], q1 = qs[1];
                uint32_t in[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                if (a.rope_cos) {
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
        }
        return;
    }
    const int r = lane & 31, hh = lane >> 5;
    const int64_t pn = L - 1;                          // fused: the new key's slot
    const bool has_new = kFused && pn < blk0 + kDecKeysPerBlock;

    if (prep && !first) __syncthreads();               // every wave has its A fragments of the last row
    // Query, weights and (fused) new-key loads, issued before the K loads and never
    // under a branch, so the waits of the staging below count the K loads exactly.
    // (An item that reuses the row's query still issues them; they are small.)
    uint4 qp0, qp1;
    uint32_t kn = 0;                                   // fused: new-key features 2 lane, 2 lane + 1
    float2 krc = {0.f, 0.f}, krs = {0.f, 0.f};         // fused: their RoPE table entries
    float4 wv;
    float wr = 0.f;
    Rope32 rope_row;                                   // fused: the token's RoPE table row (scalar loads)
    if constexpr (kFused) {
        const uint4 *qs = reinterpret_cast<const uint4 *>(a.q_bf16 + ((int64_t)qrow * LK_HEADS + head) * LK_DIM + 16 * sub);
        qp0 = qs[0];
        qp1 = qs[1];
        wr = a.w[(int64_t)qrow * LK_HEADS + head];
        kn = reinterpret_cast<const uint32_t *>(a.k_new + (int64_t)b * LK_DIM)[lane];
        // The new key's table entries are loaded whether or not RoPE is on (a load
        // under a branch would be waited for with all later loads); without tables
        // they come from the key row itself and are ignored.
        const bool rope_on = a.rope_cos != nullptr;
        const float *kc_row = rope_on ? a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2) : reinterpret_cast<const float *>(a.k_new);
        const float *ks_row = rope_on ? a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2) : reinterpret_cast<const float *>(a.k_new);
        krc = reinterpret_cast<const float2 *>(kc_row)[lane & 15];
        krs = reinterpret_cast<const float2 *>(ks_row)[lane & 15];
        if (rope_on)                                   // the step's token: shared by the query and the new key
            load_rope32_uniform(a.rope_cos + (int64_t)qrow * (LK_ROPE_DIM / 2),
                                a.rope_sin + (int64_t)qrow * (LK_ROPE_DIM / 2), rope_row);
    } else {
        qp0 = reinterpret_cast<const uint4 *>(a.q_fp8 + (int64_t)qrow * LK_HEADS * LK_DIM)[threadIdx.x];
        // Every thread loads and stores a float4 of the weights (lane % 16 picks which).
        wv = reinterpret_cast<const float4 *>(a.w_eff + (int64_t)qrow * LK_HEADS)[lane & 15];
    }
    // Key scales before the K loads: the first tile pair's store needs them, and a
    // load issued after the K loads could only be waited for together with all of K.
    float ks[kDecTiles / 2];
#pragma unroll
    for (int p = 0; p < kDecTiles / 2; p++) {
        const int64_t s = key0 + 64 * p + lane;
        ks[p] = a.k_scale[(int64_t)b * a.cache_seq_stride + (s < L ? s : 0)];
    }
    const uint8_t *kbase = a.k_cache + (int64_t)b * a.cache_seq_stride * LK_DIM;
    uint4 kv[kDecTiles][4];
    auto load_tile = [&](int j) {
        const int64_t s = key0 + 32 * j + r;
        const uint4 *src = reinterpret_cast<const uint4 *>(kbase + (s < L ? s : 0) * LK_DIM + 64 * hh);
#pragma unroll
        for (int c = 0; c < 4; c++) kv[j][c] = src[c];       // rows past L re-read row 0 (masked below)
    };
    // The fused kernel issues half of the wave's K loads before the query preparation
    // and half after it: issuing all sixteen first left waves queued behind the
    // address pipeline for thousands of cycles before their preparation could start,
    // and the block's barrier waited for the last of them (measured: 14.0 -> 12.2 us).
    constexpr int kEarlyTiles = kFused ? kDecTiles / 2 : kDecTiles;
#pragma unroll
    for (int j = 0; j < kEarlyTiles; j++) load_tile(j);
    // Keep these loads above this point, ahead of the staging and its waits.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFused) {
      if (prep) {
        uint32_t in[8] = {qp0.x, qp0.y, qp0.z, qp0.w, qp1.x, qp1.y, qp1.z, qp1.w};
        Rope16 rope;
        if (a.rope_cos) {
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
        if (has_new && wave == 0) {                    // the new key, spread over wave 0 (2 features a lane)
            uint32_t kin = kn;
            if (a.rope_cos) rope_row_wave(kin, krc, krs);
            int kj;
            const uint32_t kc = quantize_row_wave(kin, kj);
            const int64_t row = (int64_t)b * a.cache_seq_stride + pn;
            reinterpret_cast<uint16_t *>(a.k_cache + row * LK_DIM)[lane] = (uint16_t)kc;
            reinterpret_cast<uint16_t *>(snew)[lane] = (uint16_t)kc;
            if (lane == 0) {
                const float ksc = __builtin_ldexpf(1.0f, kj);
                a.k_scale[row] = ksc;
                sm.snew_scale = ksc;
            }
        }
    } else if (prep) {
        const int piece = threadIdx.x;                 // head piece / 8, 16-byte chunk piece % 8
        *reinterpret_cast<uint4 *>(sq + (piece >> 3) * kQPitch + 16 * (piece & 7)) = qp0;
        reinterpret_cast<float4 *>(sw)[lane & 15] = wv;    // duplicate stores of equal values
    }
#pragma unroll
    for (int j = kEarlyTiles; j < kDecTiles; j++) load_tile(j);
    __syncthreads();
    // A wave whose keys are all masked still runs the tiles (on re-read row 0) and
    // stores -inf: a branch here would let the compiler sink the K loads below the
    // barrier.  Only blocks that straddle a row's end have such waves.
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
#pragma unroll
    for (int p = 0; p < kDecTiles / 2; p++) {
        if (has_new) {                                 // the lanes holding the new key take the fresh codes
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                if (key0 + 32 * (2 * p + h2) + r == pn) {
#pragma unroll
                    for (int c = 0; c < 4; c++) kv[2 * p + h2][c] = snew[4 * hh + c];
                }
            }
            if (key0 + 64 * p + lane == pn) ks[p] = sm.snew_scale;
        }
        const float p0 = score_tile(kv[2 * p], f);
        const float p1 = score_tile(kv[2 * p + 1], f);
        // lanes 0-31: tile 2p, key l; lanes 32-63: tile 2p+1, key l-32  ->  key key0 + 64p + l
        const float sum = halves_sum_pair(p0, p1);
        const int64_t s = key0 + 64 * p + lane;
        if (s < T) out[s] = s < L ? sum * ks[p] : -__builtin_inff();
    }
}

template <bool kFused>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) DecodeShared sm;
    decode_item<kFused, true>(a, sm, blockIdx.y, (int64_t)blockIdx.x * kDecKeysPerBlock, true);
}

// Grids of more items than the chip runs at once (many rows, or ragged rows whose key
// blocks mostly end early): a block per compute unit walks a contiguous range of the
// valid items, in row order, so it quantizes each row's query once for all of its
// items of that row, and items of different lengths even out across blocks.  Every
// block derives the same schedule from the row lengths: row r has
// ceil(L_r / kDecKeysPerBlock) items (one for a row with L_r = 0 when the quantized
// query is requested), and the key blocks past them are swept to -inf by block r % grid.
constexpr int kPersistMaxRows = kDecThreads;
template <bool kFused>
__global__ void __launch_bounds__(kDecThreads) decode_persistent_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) DecodeShared sm;
    __shared__ int32_t first_item[kPersistMaxRows + 1];   // row r's items: first_item[r] .. first_item[r+1]-1
    __shared__ int32_t wave_tot[kDecWaves];
    const int nrows = a.rows.B * a.rows.S;             // <= kPersistMaxRows (host check)
    const int64_t T = a.rows.T;
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
    int nv = 0;
    if (tid < nrows) {
        const int64_t L = row_len(a.rows, tid / a.rows.S, tid % a.rows.S);
        nv = (int)((L + kDecKeysPerBlock - 1) / kDecKeysPerBlock);
        if (kFused && L == 0 && a.q_fp8_out) nv = 1;
    }
    // exclusive scan of nv over the rows (one per thread)
    int incl = nv;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int w = 0; w < kDecWaves; w++) base += w < wave ? wave_tot[w] : 0;
    first_item[tid] = base + incl - nv;
    if (tid == kDecThreads - 1) first_item[kDecThreads] = base + incl;
    __syncthreads();
    const int total = first_item[kDecThreads];
    const int G = gridDim.x, g = blockIdx.x;
    // -inf for the key blocks past each row's items
    for (int r = g; r < nrows; r += G) {
        const int64_t s0 = (int64_t)(first_item[r + 1] - first_item[r]) * kDecKeysPerBlock;
        float *out = a.scores + (int64_t)r * T;
        for (int64_t s = s0 + tid; s < T; s += kDecThreads) out[s] = -__builtin_inff();
    }
    const int i0 = (int)((int64_t)total * g / G), i1 = (int)((int64_t)total * (g + 1) / G);
    int row = 0;
    {                                                  // the row of item i0 (binary search)
        int lo = 0, hi = nrows - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first_item[mid] <= i0) lo = mid; else hi = mid - 1;
        }
        row = lo;
    }
    int prev = -1;
    for (int it = i0; it < i1; it++) {
        while (first_item[row + 1] <= it) row++;
        const int64_t blk0 = (int64_t)(it - first_item[row]) * kDecKeysPerBlock;
        if (row != prev) decode_item<kFused, true>(a, sm, row, blk0, it == i0);
        else decode_item<kFused, false>(a, sm, row, blk0, false);
        prev = row;
    }
}

// ------------------------------------------------------------------ prefill (S > 1)
// A block of 4 waves (one per SIMD) owns 4 consecutive query tokens of one sequence
// (one per wave) and a slice of 2048 keys, taken as sixteen chunks of 128.  Each
// chunk is read from HBM once per block, converted to f16 once and kept in LDS, where
// every wave streams it through the MFMA against its own query held in registers.
// The chunks are double buffered: the loads of chunk c+1 are issued before chunk c's
// MFMA work and land in the other LDS buffer after it, and the query is loaded and
// converted once per slice.  Two blocks share a CU (70 KB of LDS each), so each SIMD
// runs one wave of each: the two never meet at a barrier, and one block's prologue
// and chunk hand-overs are covered by the other block's MFMA work.  (With both waves
// of a SIMD in one block, the issue arbiter's preference for the older wave made the
// younger one finish each chunk ~40% later while the block waited at the barrier.)
constexpr int kPreWaves = 4;
constexpr int kPreThreads = 64 * kPreWaves;
constexpr int kPreChunk = 128;                      // keys per LDS buffer
constexpr int kPreChunks = 16;                      // chunks per block
constexpr int kPreSlice = kPreChunk * kPreChunks;   // keys per block
constexpr int kPreRowBytes = 2 * LK_DIM + 16;       // f16 row + 16 B pad against bank conflicts
static_assert(kPreThreads == 2 * kPreChunk, "two threads stage each key row");

// One thread's share of a chunk in flight: half a key row (64 fp8 bytes) and, for
// threads below kPreChunk, one key scale.
struct ChunkPart {
    uint4 v[4];
    float ks;
};

__device__ __forceinline__ void load_chunk_part(const uint8_t *__restrict__ kbase, const float *__restrict__ sbase,
                                                int64_t kc, int64_t Lmax, ChunkPart &p) {
    const int kr = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t s = kc + kr;
    if (s < Lmax) {
        const uint4 *src = reinterpret_cast<const uint4 *>(kbase + s * LK_DIM + 64 * half);
#pragma unroll
        for (int c = 0; c < 4; c++) p.v[c] = src[c];
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) p.v[c] = make_uint4(0, 0, 0, 0);
    }
    p.ks = (threadIdx.x < kPreChunk && kc + threadIdx.x < Lmax) ? sbase[kc + threadIdx.x] : 0.0f;
}

__device__ __forceinline__ void store_chunk_part(uint8_t *sk, float *sks, const ChunkPart &p) {
    const int kr = threadIdx.x >> 1, half = threadIdx.x & 1;
    half8 *dst = reinterpret_cast<half8 *>(sk + kr * kPreRowBytes + 128 * half);
#pragma unroll
    for (int c = 0; c < 4; c++) {
        dst[2 * c] = fp8x8_to_half8(p.v[c].x, p.v[c].y);
        dst[2 * c + 1] = fp8x8_to_half8(p.v[c].z, p.v[c].w);
    }
    if (threadIdx.x < kPreChunk) sks[threadIdx.x] = p.ks;
}

__global__ void __launch_bounds__(kPreThreads)
score_prefill_kernel(const uint8_t *__restrict__ q_fp8, const float *__restrict__ w_eff,
                     const uint8_t *__restrict__ k_cache, const float *__restrict__ k_scale,
                     int64_t cache_seq_stride, RowsDev rows, float *__restrict__ scores) {
    __shared__ __attribute__((aligned(16))) uint8_t sk[2][kPreChunk * kPreRowBytes];
    __shared__ float sks[2][kPreChunk];
    const int lane = __lane_id();
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.z;
    // Row groups in reverse: under a causal mask the longest rows start first, so the
    // heaviest blocks do not trail at the end of the launch.
    const int t0 = (gridDim.y - 1 - blockIdx.y) * kPreWaves;
    const int64_t T = rows.T;
    const int64_t slice0 = (int64_t)blockIdx.x * kPreSlice;
    const int t = t0 + wave;
    const bool has_row = t < rows.S;
    const int64_t L = has_row ? row_len(rows, b, t) : 0;
    // The block needs keys below the largest valid length of its rows.
    const int t_last = (t0 + kPreWaves - 1 < rows.S ? t0 + kPreWaves - 1 : rows.S - 1);
    const int64_t Lmax = row_len(rows, b, t_last);     // row_len is non-decreasing in t
    float *out = scores + ((int64_t)b * rows.S + t) * T;
    // Chunks of the slice with any valid key for some row of the block.
    const int64_t live = Lmax - slice0;
    const int nchunks = live <= 0 ? 0 : (live >= kPreSlice ? kPreChunks : (int)((live + kPreChunk - 1) / kPreChunk));
    // -inf for this row's slots of the chunks no row of the block needs.
    if (has_row)
        for (int64_t s = slice0 + (int64_t)nchunks * kPreChunk + lane; s < slice0 + kPreSlice && s < T; s += 64)
            out[s] = -__builtin_inff();
    if (nchunks == 0) return;

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
    for (int c = 0; c < nchunks; c++) {
        const int64_t kc = slice0 + (int64_t)c * kPreChunk;
        const bool more = c + 1 < nchunks;
        if (more) load_chunk_part(kbase, sbase, kc + kPreChunk, Lmax, part);   // in flight during the MFMA work
        const uint8_t *skc = sk[c & 1];
        const float *sksc = sks[c & 1];
        if (has_row && kc + kPreChunk <= L) {
            // Every key of the chunk is valid for this row: a software pipeline in which
            // the MFMA chain of tile j+1 is issued before the ReLU / weighted-sum epilogue
            // of tile j, so the VALU epilogue runs in the shadow of the matrix core.
            const uint8_t *rowbase = skc + r * kPreRowBytes + 128 * hh;
            auto mfma_tile = [&](int j, float16v acc[2]) {
                acc[0] = float16v{};
                acc[1] = float16v{};
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    const half8 bk = *reinterpret_cast<const half8 *>(rowbase + 32 * j * kPreRowBytes + 16 * kk);
#pragma unroll
                    for (int m = 0; m < 2; m++)
                        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[m][kk], bk, acc[m], 0, 0, 0);
                }
            };
            float16v acc[2][2];
            float p[2];
            mfma_tile(0, acc[0]);
#pragma unroll
            for (int j = 0; j < kPreChunk / 32; j++) {
                // One scheduling region per stage: the next tile's 8 operand reads first,
                // then part of this tile's epilogue while they land, then the MFMA chain
                // interleaved with the rest of the epilogue (two MFMAs, six VALU ops per
                // K-step).
                __builtin_amdgcn_sched_barrier(0);
                if (j + 1 < kPreChunk / 32) mfma_tile(j + 1, acc[(j + 1) & 1]);
                p[j & 1] = relu_weighted_sum(acc[j & 1], f);
                if (j & 1) {
                    const float sum = halves_sum_pair(p[0], p[1]);
                    const int64_t s = kc + 32 * (j - 1) + lane;
                    out[s] = sum * sksc[32 * (j - 1) + lane];   // s < L <= T
                }
                if (j + 1 < kPreChunk / 32) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);       // the tile's 8 operand reads
                    __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);      // VALU while they land
#pragma unroll
                    for (int kk = 0; kk < 8; kk++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        } else if (has_row) {
            for (int j = 0; j < kPreChunk / 32; j += 2) {
                if (kc + 32 * j >= L) {                // rest of this chunk is masked for the row
                    for (int64_t s = kc + 32 * j + lane; s < kc + kPreChunk && s < T; s += 64) out[s] = -__builtin_inff();
                    break;
                }
                float partial[2];
#pragma unroll
                for (int jj = 0; jj < 2; jj++) {
                    const uint8_t *row = skc + (32 * (j + jj) + r) * kPreRowBytes + 128 * hh;
                    float16v acc[2] = {};
#pragma unroll
                    for (int kk = 0; kk < 8; kk++) {
                        const half8 bk = *reinterpret_cast<const half8 *>(row + 16 * kk);
#pragma unroll
                        for (int m = 0; m < 2; m++)
                            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[m][kk], bk, acc[m], 0, 0, 0);
                    }
                    partial[jj] = relu_weighted_sum(acc, f);
                }
                const float sum = halves_sum_pair(partial[0], partial[1]);
                const int64_t s = kc + 32 * j + lane;
                if (s < T) out[s] = s < L ? sum * sksc[32 * j + lane] : -__builtin_inff();
            }
        }
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
// once; beyond, the persistent form with one block per compute unit.
template <bool kFused>
hipError_t launch_decode_grid(const DecodeArgs &a, hipStream_t stream) {
    const RowsDev &rows = a.rows;
    const int64_t nblk = (rows.T + kDecKeysPerBlock - 1) / kDecKeysPerBlock;
    const int64_t nrows = (int64_t)rows.B * rows.S;
    const int cus = cu_count();
    if (nrows <= kPersistMaxRows && nblk * nrows * 4 > (int64_t)cus * 5) {
        const unsigned grid = (unsigned)(nblk * nrows < cus ? nblk * nrows : cus);
        return launch(decode_persistent_kernel<kFused>, dim3(grid), dim3(kDecThreads), 0u, stream, a);
    }
    dim3 grid((unsigned)nblk, (unsigned)rows.B);
    return launch(decode_kernel<kFused>, grid, dim3(kDecThreads), 0u, stream, a);
}

}  // namespace

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
        dim3 grid((unsigned)((rows.T + kPreSlice - 1) / kPreSlice), (unsigned)((rows.S + kPreWaves - 1) / kPreWaves),
                  (unsigned)rows.B);
        return launch(score_prefill_kernel, grid, dim3(kPreThreads), 0u, stream, q_fp8, w_eff, k_cache,
                      k_scale, cache_seq_stride, rows, scores);
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

}  // namespace lk

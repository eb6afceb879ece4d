// mla.hip -- sparse MLA decode attention over the indexer's selected keys (gfx950).
//
// Page "Join query parts" (the MQA-decode excerpt): for one decode token of sequence
// b and head h, logits s_t = scale * (qc_h . c_t + qr_h . r_t) over the cached latent
// rows c_t (512 features) and rotary rows r_t (64 features), the index mask leaves
// only the top-k selected slots t in I, p = softmax(s) over I, o_h = sum_t p_t c_t
// (512 features; the up-projection that follows is outside this path).
//
// Split kernel: block (split, head half, b) owns 64 heads and one split of at most
// 256 entries of the row's index list, taken as chunks of 32 keys.  A chunk's latent
// (1 KB) and rotary (128 B) rows are gathered from HBM straight into LDS by DMA
// (global_load_lds: one instruction moves one latent row, or eight rotary rows),
// key-major, each row's 16-byte chunks XOR-swizzled by a pattern of the row index
// through the source address.  Four chunk buffers rotate; chunk c + 2 is in flight
// while chunk c is scored and chunk c - 1 is multiplied into o.
// Eight waves, two per SIMD, in two roles:
//  - score waves (0..3): wave a holds the query of heads 16a .. 16a+15 (576 features,
//    bf16, 72 registers) and computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 for
//    all 32 keys of the chunk (two key tiles), so that each lane holds 8 keys of one
//    head and the four lanes of a head settle its chunk max by two lane swaps: the
//    softmax needs no other wave, and one barrier per chunk suffices.  Each wave
//    writes p (bf16) for its heads and keeps per-lane partial sums l, added up once
//    at the end.  The key rows are read from LDS by all four score waves.
//  - P V waves (4..7): wave v accumulates o for all 64 heads and latent features
//    128v .. 128v+127 (128 registers) with v_mfma_f32_32x32x16_bf16, A = p from LDS
//    (two 32-head tiles), B = 8 consecutive keys of one feature per lane, read from the
//    key-major rows by two transposing LDS reads (ds_read_b64_tr_b16: within 16 lanes,
//    lane l receives element l % 4 of the 8-byte pieces read by lanes 4i + l / 4).
//    These reads run at about a quarter of the rate of 16-byte LDS reads (measured),
//    so each B operand feeds both head tiles.  The P V waves also issue the chunk DMAs.
// The block's query (64 heads x 576 features, 72 KB) goes by DMA into chunk buffers 2
// and 3 (one instruction per 1 KB latent row), each score wave moving its own 16 heads,
// and is read into registers before chunks 2 and 3 overwrite those buffers; the first
// two chunks' gathers run meanwhile.
// The split writes its unnormalised o with the running max m (base-2 logit units)
// and sum l to the workspace.
// Combine kernel: per (b, h), o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
#include <atomic>
#include <mutex>

#include "lk_device.h"

namespace lk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kH = LK_MLA_HEADS;          // 128
constexpr int kDc = LK_MLA_LATENT;        // 512
constexpr int kDr = LK_MLA_ROPE;          // 64
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerBlock = 64;
constexpr int kChunk = 32;                    // keys per LDS chunk
constexpr int kSplit = 256;                   // index-list entries per block
constexpr int kBufs = 4;                      // chunk buffers in LDS
constexpr int kLatRow = 2 * kDc;              // bytes per latent row in LDS (64 chunks of 16 B)
constexpr int kRopeRow = 2 * kDr;             // bytes per rotary row in LDS (8 chunks of 16 B)
constexpr int kPPitch = kChunk + 8;           // bf16 per head row of p (80 B: conflict-free reads)

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

// bf16 (nearest-even) bits of two floats, a in the low half: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}


// XOR pattern of latent row r: r % 16 rotated right by one bit.  Reads of one chunk
// position from 16 consecutive rows (the S operand, ds_read_b128) then hit 16 distinct
// 16-byte slots at the full LDS rate; the transposing reads of the P V operand run at
// about a quarter of that rate whatever the pattern (measured), this one included.
__device__ __forceinline__ int lat_swizzle(int r) { return ((r & 1) << 3) | ((r >> 1) & 7); }

// Gather chunk c (keys sidx[32c .. 32c+31]) into lat / rope; issued by the P V waves,
// whose phases have slack: P V wave v moves latent rows 8v .. 8v+7 (one DMA each) and
// rotary rows 8v .. 8v+7 (one DMA).  Row r's 16-byte chunk j lands in slot
// j ^ lat_swizzle(r) (latent) or j ^ (r % 8) (rotary).
constexpr int kDma = 9;                        // DMA instructions per chunk per P V wave
__device__ __forceinline__ void gather_chunk(const MlaArgs &a, int b, const int32_t *sidx, int c, uint8_t *lat,
                                             uint8_t *rope, int v, int lane) {
    const int4 r0 = *reinterpret_cast<const int4 *>(&sidx[c * kChunk + 8 * v]);
    const int4 r1 = *reinterpret_cast<const int4 *>(&sidx[c * kChunk + 8 * v + 4]);
    const int rr = sidx[c * kChunk + 8 * v + (lane >> 3)];
    const int rows[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    const uint8_t *kl = reinterpret_cast<const uint8_t *>(a.kv_lat) + (int64_t)b * a.stride * kLatRow;
    const uint8_t *kr = reinterpret_cast<const uint8_t *>(a.kv_rope) + (int64_t)b * a.stride * kRopeRow;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int r = 8 * v + j;
        const int64_t row = rows[j] < 0 ? 0 : rows[j];
        dma_b128(kl + row * kLatRow + 16 * (lane ^ lat_swizzle(r)), lat + r * kLatRow);
    }
    const int r = 8 * v + (lane >> 3);
    const int64_t row = rr < 0 ? 0 : rr;
    dma_b128(kr + row * kRopeRow + 16 * ((lane & 7) ^ (r & 7)), rope + 8 * v * kRopeRow);
}

// Query staging: head hh (0 .. 63) of the block goes to buffer 2 + hh / 32, row
// r = hh % 32; latent 16-byte chunk j in slot j ^ lat_swizzle(r), rotary chunk j in
// slot j ^ ((r / 2) % 8) (16 rows of a register read hit distinct banks).  Score wave w
// moves heads 16w .. 16w+15: one DMA per latent row, one per eight rotary rows.
__device__ __forceinline__ int qrope_swizzle(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ void stage_query(const MlaArgs &a, int b, int half, uint8_t (*lat)[kChunk * kLatRow],
                                            uint8_t (*rope)[kChunk * kRopeRow], int w, int lane) {
    const int64_t h0 = (int64_t)b * kH + half * kHeadsPerBlock;
    const uint8_t *ql = reinterpret_cast<const uint8_t *>(a.q_lat) + h0 * kLatRow;
    const uint8_t *qr = reinterpret_cast<const uint8_t *>(a.q_rope) + h0 * kRopeRow;
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int hh = 16 * w + j, r = hh & 31;
        dma_b128(ql + hh * kLatRow + 16 * (lane ^ lat_swizzle(r)), lat[2 + (hh >> 5)] + r * kLatRow);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int hh0 = 16 * w + 8 * i, hh = hh0 + (lane >> 3), r = hh & 31;
        dma_b128(qr + hh * kRopeRow + 16 * ((lane & 7) ^ qrope_swizzle(r)), rope[2 + (hh0 >> 5)] + (hh0 & 31) * kRopeRow);
    }
}

// Raise the running max only when a chunk exceeds it by more than 2^8 (base-2 logits):
// p = 2^(x - m) then stays below 2^8, and the rescale of o runs on few chunks.  The
// result does not depend on which m is used.
constexpr float kLazyMax = 8.f;

struct SharedMem {
    uint8_t lat[kBufs][kChunk * kLatRow];     // 128 KB
    uint8_t rope[kBufs][kChunk * kRopeRow];   // 16 KB
    uint16_t p[2][kHeadsPerBlock * kPPitch];  // p of the chunk last scored, bf16 [head][key]
    float alpha[2][kHeadsPerBlock];           // o rescale factor per head for that chunk
    int32_t rescale[2][4];                    // any alpha != 1, per score wave (16 heads)
    int32_t sidx[kSplit];
};

// ---- score wave: S^T = K Q^T for 32 keys x 16 heads, softmax bookkeeping
struct ScoreState {
    bf16x8 qa[18];                            // B operand per K-step (features 32k .. 32k+31; k >= 16: rotary)
    uint32_t off_lat[4], off_rope[2];         // swizzled LDS offsets (see score_chunk)
    float m, l;                               // head 16 wave + r16; l: this lane's keys only
};

// Lanes r16, r16 + 16, r16 + 32, r16 + 48 hold the same head: combine their values.
__device__ __forceinline__ float max4_groups(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));          // groups (0, 1) and (2, 3)
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum4_groups(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Scores and softmax of chunk c for score wave a: lane (r16, g4) holds keys
// 16kt + 4g4 + i (kt = 0, 1; i = 0..3) of head 16a + r16, so a head's chunk max, its
// running max and its p all stay within the wave.  Writes p (bf16) and alpha into
// buffer pbuf for the P V waves.
__device__ __forceinline__ void score_chunk(ScoreState &st, SharedMem &sm, int buf, int c, int pbuf, int wave,
                                            int lane, float sl2) {
    const int r16 = lane & 15, g4 = lane >> 4;
    const uint8_t *lat = sm.lat[buf];
    const uint8_t *rope = sm.rope[buf];
    // Two accumulators per key tile (even and odd K-steps): four independent chains
    // of dependent products keep the matrix pipeline busy.
    f32x4 s2[2][2] = {};
    // A operand of K-step k, key tile kt: key 16kt + r16, features 32k + 8 g4 .. +7;
    // chunk 16 j + c' of a row lies 256 j bytes after chunk c' (the XOR only touches
    // the low 4 bits, and it depends on the row's low 4 bits only).  The reads run
    // kAhead K-steps ahead of the products (the order is pinned: one score wave per
    // SIMD has nothing else to hide the LDS latency behind).
    constexpr int kAhead = 6;
    bf16x8 kb[18][2];
    auto read = [&](int k) {
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            const uint8_t *p0 = k < 16 ? lat + kt * 16 * kLatRow + st.off_lat[k % 4] + 256 * (k / 4)
                                       : rope + kt * 16 * kRopeRow + st.off_rope[k - 16];
            kb[k][kt] = as_bf16x8(*reinterpret_cast<const uint4 *>(p0));
        }
    };
#pragma unroll
    for (int k = 0; k < kAhead; k++) read(k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 18; k++) {
        if (k + kAhead < 18) read(k + kAhead);
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
            s2[kt][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[k][kt], st.qa[k], s2[kt][k & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    const f32x4 s[2] = {s2[0][0] + s2[0][1], s2[1][0] + s2[1][1]};
    float x[2][4];
    float cm = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        const int4 ids = *reinterpret_cast<const int4 *>(&sm.sidx[c * kChunk + 16 * kt + 4 * g4]);
        const bool ok[4] = {ids.x >= 0, ids.y >= 0, ids.z >= 0, ids.w >= 0};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            x[kt][i] = ok[i] ? s[kt][i] * sl2 : -__builtin_inff();
            cm = fmaxf(cm, x[kt][i]);
        }
    }
    cm = max4_groups(cm);                                       // chunk max of the head
    float alpha = 1.f;
    bool up = false;
    if (cm > st.m + kLazyMax) {                                 // also when m is -inf and cm is finite
        alpha = __builtin_amdgcn_exp2f(st.m - cm);              // 0 when m was -inf
        // While m is -inf every p so far is 0, so o is still 0: no rescale is needed
        // (this spares the P V waves a pass over o after the first chunk).
        up = st.m != -__builtin_inff();
        st.m = cm;
    }
    // m is -inf only while every key so far is masked: then p = 2^(-inf) = 0
    const float mref = st.m == -__builtin_inff() ? 0.f : st.m;
    const int hb = 16 * wave + r16;                             // head within the block
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; i++) e[i] = __builtin_amdgcn_exp2f(x[kt][i] - mref);
        const uint32_t w01 = bf16_pair(e[0], e[1]), w23 = bf16_pair(e[2], e[3]);
        sum += __uint_as_float(w01 << 16);
        sum += __uint_as_float(w01 & 0xFFFF0000u);
        sum += __uint_as_float(w23 << 16);
        sum += __uint_as_float(w23 & 0xFFFF0000u);
        *reinterpret_cast<uint2 *>(&sm.p[pbuf][hb * kPPitch + 16 * kt + 4 * g4]) = make_uint2(w01, w23);
    }
    st.l = st.l * alpha + sum;
    if (g4 == 0) sm.alpha[pbuf][hb] = alpha;
    const bool wany = __any(up);
    if (lane == 0) sm.rescale[pbuf][wave] = wany;
}

// ---- P V wave: o[64 heads][128 features] += P V
struct PvState {
    float o[2][4][16];                        // [head tile][feature tile][register]
    uint32_t off[2][4];                       // transposing-read offsets [h'][feature tile]
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// o = alpha o + P V for chunk `buf` with p and alpha from `pbuf`.  The rescale flags
// (and alpha, where a head group needs it) are read first; every other LDS read of the
// chunk (p for both K-steps, 16 transposing reads) is issued next, in pinned order, so
// that the rescale and the first products wait only for the reads they use.
__device__ __forceinline__ void pv_chunk(PvState &st, const SharedMem &sm, int buf, int pbuf, int lane) {
    const uint8_t *lat = sm.lat[buf];
    const int4 fl = *reinterpret_cast<const int4 *>(&sm.rescale[pbuf][0]);
    const bool res[2] = {(fl.x | fl.y) != 0, (fl.z | fl.w) != 0};   // head tile mt = score waves 2mt, 2mt + 1
    // register i of a tile holds head row 8 (i / 4) + 4 (lane / 32) + i % 4
    float al[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        if (!res[mt]) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float4 v = *reinterpret_cast<const float4 *>(&sm.alpha[pbuf][32 * mt + 8 * j + 4 * (lane >> 5)]);
            al[mt][4 * j] = v.x;
            al[mt][4 * j + 1] = v.y;
            al[mt][4 * j + 2] = v.z;
            al[mt][4 * j + 3] = v.w;
        }
    }
    // A: head 32 mt + lane % 32, keys 16 ks + 8 (lane / 32) .. +7
    bf16x8 pa[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
            pa[ks][mt] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                &sm.p[pbuf][(32 * mt + (lane & 31)) * kPPitch + 16 * ks + 8 * (lane >> 5)]));
    v4i16 hv[2][4][2];
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int n = 0; n < 4; n++)
#pragma unroll
            for (int h = 0; h < 2; h++)
                hv[ks][n][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16 *)(lptr_t)(lat + st.off[h][n] + ks * 16 * kLatRow));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        if (!res[mt]) continue;
#pragma unroll
        for (int n = 0; n < 4; n++)
#pragma unroll
            for (int i = 0; i < 16; i++) st.o[mt][n][i] *= al[mt][i];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int n = 0; n < 4; n++) {
            const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[ks][n][0], hv[ks][n][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                f32x16 acc;
#pragma unroll
                for (int i = 0; i < 16; i++) acc[i] = st.o[mt][n][i];
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks][mt], vb, acc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 16; i++) st.o[mt][n][i] = acc[i];
            }
        }
}

// Block-level context shared by both roles.
struct SplitCtx {
    int b, split, half, nch, nk, k0, wave, lane;
    float sl2;
};

// Barrier sequence, identical in both roles: slot list filled (the score waves' query
// DMAs are in flight), chunks 0 and 1 issued with chunk 0 and the query landed, query
// read into registers, then one per iteration c = 0 .. nch (p of chunk c written,
// chunk c + 1 landed).  Iteration c scores chunk c and multiplies chunk c - 1; the DMA
// of chunk c + 2 goes into the buffer of chunk c - 2, free since iteration c - 1
// (chunk 2's, into the query staging, goes once the query is in registers).  The P V
// waves issue no global loads but their DMAs, so vmcnt counts exactly those.

__device__ __forceinline__ void score_role(const MlaArgs &a, SharedMem &sm, const SplitCtx &x) {
    const int r16 = x.lane & 15, g4 = x.lane >> 4;
    ScoreState ss;
    stage_query(a, x.b, x.half, sm.lat, sm.rope, x.wave, x.lane);
    ss.m = -__builtin_inff();
    ss.l = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) ss.off_lat[kk] = r16 * kLatRow + 16 * ((4 * kk + g4) ^ lat_swizzle(r16));
#pragma unroll
    for (int kk = 0; kk < 2; kk++) ss.off_rope[kk] = r16 * kRopeRow + 16 * ((4 * kk + g4) ^ (r16 & 7));
    __syncthreads();                                           // slot list
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                  // this wave's query DMAs
    __syncthreads();                                           // chunk 0 and the query in LDS
    // Query fragments of head 16 wave + r16, which this wave staged itself: row
    // 16 (wave % 2) + r16 of buffer 2 + wave / 2.
    {
        const int r = 16 * (x.wave & 1) + r16;
        const uint8_t *ql = sm.lat[2 + (x.wave >> 1)] + r * kLatRow;
        const uint8_t *qr = sm.rope[2 + (x.wave >> 1)] + r * kRopeRow;
#pragma unroll
        for (int k = 0; k < 16; k++)
            ss.qa[k] = as_bf16x8(*reinterpret_cast<const uint4 *>(ql + 16 * ((4 * k + g4) ^ lat_swizzle(r))));
#pragma unroll
        for (int k = 0; k < 2; k++)
            ss.qa[16 + k] = as_bf16x8(*reinterpret_cast<const uint4 *>(qr + 16 * ((4 * k + g4) ^ qrope_swizzle(r))));
    }
    __syncthreads();                                           // query in registers
    for (int c = 0; c <= x.nch; c++) {
        if (c < x.nch) score_chunk(ss, sm, c % kBufs, c, c & 1, x.wave, x.lane, x.sl2);
        __syncthreads();                                       // p of chunk c, chunk c + 1 in LDS
    }
    const float l = sum4_groups(ss.l);
    if (g4 == 0) {
        float *mp = a.ml_part + (((int64_t)x.b * a.nsplit + x.split) * kH + x.half * kHeadsPerBlock + 16 * x.wave + r16) * 2;
        mp[0] = ss.m;
        mp[1] = l;
    }
}

__device__ __forceinline__ void pv_role(const MlaArgs &a, SharedMem &sm, const SplitCtx &x) {
    const int lane = x.lane, r16 = lane & 15;
    const int v = x.wave - 4;
    PvState ps;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int n = 0; n < 4; n++)
#pragma unroll
            for (int i = 0; i < 16; i++) ps.o[mt][n][i] = 0.f;
    // Transposing read h' for feature tile n, K-step ks: source lane s = lane % 16 of
    // 16-lane group q = lane / 16 points at key row 16 ks + 8 (q / 2) + 4 h' + s / 4,
    // features 128 v + 32 n + 16 (q % 2) + 4 (s % 4) .. +3, so lane r of the group
    // receives feature ... + r, keys ... + 4h' + i.  The row's low 4 bits do not depend
    // on ks: offsets differ by 16 KB per ks.
    {
        const int q = lane >> 4, sq = r16 & 3;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int row = 8 * (q >> 1) + 4 * h + (r16 >> 2);
#pragma unroll
            for (int n = 0; n < 4; n++) {
                const int ch = 16 * v + 4 * n + 2 * (q & 1) + (sq >> 1);
                ps.off[h][n] = row * kLatRow + 16 * (ch ^ lat_swizzle(row)) + 8 * (sq & 1);
            }
        }
    }
    // This split's slice of the index list; unused or out-of-range entries become -1.
    {
        const int i = threadIdx.x - 256;
        const int v0 = i < x.nk ? a.idx[(int64_t)x.b * a.n_idx + x.k0 + i] : -1;
        sm.sidx[i] = (v0 >= 0 && v0 < a.cap) ? v0 : -1;
    }
    __syncthreads();                                           // slot list
    gather_chunk(a, x.b, sm.sidx, 0, sm.lat[0], sm.rope[0], v, lane);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                  // chunk 0
    if (x.nch > 1) gather_chunk(a, x.b, sm.sidx, 1, sm.lat[1], sm.rope[1], v, lane);
    __syncthreads();                                           // chunk 0 in LDS
    __syncthreads();                                           // query in registers
    if (x.nch > 2) gather_chunk(a, x.b, sm.sidx, 2, sm.lat[2], sm.rope[2], v, lane);
    for (int c = 0; c <= x.nch; c++) {
        const bool more = c + 2 < x.nch;
        if (more && c > 0) gather_chunk(a, x.b, sm.sidx, c + 2, sm.lat[(c + 2) % kBufs], sm.rope[(c + 2) % kBufs], v, lane);
        if (c >= 1) {
            pv_chunk(ps, sm, (c - 1) % kBufs, (c - 1) & 1, lane);
        }
        if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDma)); // chunk c + 1 (all but c + 2's DMAs)
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();                                       // p of chunk c, chunk c + 1 in LDS
    }
    // register i of a tile holds head row 8 (i / 4) + 4 (lane / 32) + i % 4, feature lane % 32
    float *op = a.o_part + (((int64_t)x.b * a.nsplit + x.split) * kH + x.half * kHeadsPerBlock) * kDc + 128 * v + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int n = 0; n < 4; n++)
#pragma unroll
            for (int i = 0; i < 16; i++)
                op[(int64_t)(32 * mt + 8 * (i / 4) + 4 * (lane >> 5) + (i % 4)) * kDc + 32 * n] = ps.o[mt][n][i];
}

// Workgroups are dealt to the eight XCDs in turn (block i to XCD i % 8), and each XCD
// has its own L2.  Renumbering so that XCD k runs the consecutive logical blocks
// k n / 8 .. (k + 1) n / 8 - 1 keeps the blocks of one sequence, which read the same
// query and key rows, on one L2.  Grids whose size is not a multiple of 8 keep the
// hardware order.
__device__ __forceinline__ int xcd_local_block() {
    const int n = gridDim.x, i = blockIdx.x;
    return (n & 7) ? i : (i & 7) * (n >> 3) + (i >> 3);
}

// Logical block (b, head half, split), split fastest.
__global__ void __launch_bounds__(kThreads) mla_split_kernel(MlaArgs a) {
    __shared__ __attribute__((aligned(16))) SharedMem sm;
    LK_POISON_LDS_OBJS(sm);
    SplitCtx x;
    const int id = xcd_local_block();
    x.split = id % a.nsplit;
    x.half = (id / a.nsplit) & 1;
    x.b = id / (2 * a.nsplit);
    x.lane = __lane_id();
    x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    x.sl2 = a.scale * 1.4426950408889634f;                     // logits in base-2 units
    x.k0 = x.split * kSplit;
    x.nk = min(kSplit, a.n_idx - x.k0);                        // >= 1 by the grid
    x.nch = (x.nk + kChunk - 1) / kChunk;
    if (x.wave < 4) score_role(a, sm, x);
    else pv_role(a, sm, x);
}

// One block per (b, two heads), XCD-local like the split kernel so that the partial
// results of a sequence are read on the L2 that wrote them: 128 threads x 4 features
// per head.  Splits are taken
// eight at a time with every load of the group issued together (out-of-range splits
// read the last one and get weight 0), merged into a running max / sum.
__global__ void __launch_bounds__(256) mla_combine_kernel(MlaArgs a) {
    const int id = xcd_local_block();
    const int h = 2 * (id % (kH / 2)) + (threadIdx.x >> 7), b = id / (kH / 2);
    const int f = 4 * (threadIdx.x & 127);
    float M = -__builtin_inff(), den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < a.nsplit; s0 += 8) {
        float ms[8], ls[8];
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int64_t row = ((int64_t)b * a.nsplit + min(s0 + j, a.nsplit - 1)) * kH + h;
            const float2 ml = *reinterpret_cast<const float2 *>(a.ml_part + row * 2);
            ms[j] = s0 + j < a.nsplit ? ml.x : -__builtin_inff();
            ls[j] = ml.y;
            v[j] = *reinterpret_cast<const float4 *>(a.o_part + row * kDc + f);
        }
        float gm = M;
#pragma unroll
        for (int j = 0; j < 8; j++) gm = fmaxf(gm, ms[j]);
        if (gm == -__builtin_inff()) continue;                  // nothing valid yet
        const float r = exp2f(M - gm);                          // 0 when M was -inf
        den *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float w = exp2f(ms[j] - gm);                  // 0 for empty or padding splits
            den += w * ls[j];
            acc.x += w * v[j].x;
            acc.y += w * v[j].y;
            acc.z += w * v[j].z;
            acc.w += w * v[j].w;
        }
        M = gm;
    }
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    if (den > 0.f) res = make_float4(acc.x / den, acc.y / den, acc.z / den, acc.w / den);
    *reinterpret_cast<float4 *>(a.out + ((int64_t)b * kH + h) * kDc + f) = res;
}

}  // namespace

// Both grids are one-dimensional; a dispatch counts at most 2^32 - 1 work-items per axis.
bool mla_grid_fits(int32_t B, int32_t n_idx) {
    const int64_t nsplit = (n_idx + kSplit - 1) / kSplit;
    return nsplit * (kH / kHeadsPerBlock) * B * kThreads <= 0xFFFFFFFFLL && (int64_t)(kH / 2) * B * 256 <= 0xFFFFFFFFLL;
}

size_t mla_workspace_bytes(int32_t B, int32_t n_idx) {
    const int64_t nsplit = (n_idx + kSplit - 1) / kSplit;
    return (size_t)B * nsplit * kH * (kDc + 2) * sizeof(float);
}

// ---- The allocation-free variant's workspace: one static buffer per device, sized for
// up to kMlaScratchBytes of per-split partials (B * ceil(n_idx / 256) * 128 * 514 floats;
// 16 rows of 2048 entries take 33.7 MB).  Each device holds its own copy from module
// load until the process ends.  In host code `scratch` names a host-side stand-in, so
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kMlaScratchBytes = (size_t)LK_MLA_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kMlaScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (which must be current), or nullptr if
// the runtime cannot provide it.
void *scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
        g_scratch_dev[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

size_t mla_scratch_capacity() { return kMlaScratchBytes; }

hipError_t launch_sparse_mla_static(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *kv_lat,
                                    const uint16_t *kv_rope, int64_t stride, int64_t cap, const int32_t *idx,
                                    int32_t B, int32_t n_idx, float scale, float *out, hipStream_t stream);

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
    if (cap == 0) a.nsplit = 0;                               // no valid slot: every output row is zero
    if (a.nsplit > 0) {
        hipError_t e = launch(mla_split_kernel, dim3((unsigned)(a.nsplit * (kH / kHeadsPerBlock) * B)),
                              dim3(kThreads), 0u, stream, a);
        if (e != hipSuccess) return e;
    }
    return launch(mla_combine_kernel, dim3((unsigned)(kH / 2 * B)), dim3(256), 0u, stream, a);
}

// The same launches with the static per-device workspace (see scratch_address); the
// host checks that the request fits kMlaScratchBytes before calling this.
hipError_t launch_sparse_mla_static(const uint16_t *q_lat, const uint16_t *q_rope, const uint16_t *kv_lat,
                                    const uint16_t *kv_rope, int64_t stride, int64_t cap, const int32_t *idx,
                                    int32_t B, int32_t n_idx, float scale, float *out, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    void *ws = scratch_address(dev);
    if (!ws) return hipErrorInvalidSymbol;
    return launch_sparse_mla(q_lat, q_rope, kv_lat, kv_rope, stride, cap, idx, B, n_idx, scale, out, ws, stream);
}

}  // namespace lk

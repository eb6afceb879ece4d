// topk_device.h -- the per-row top-k of the index scores as block-level device code
// (gfx950), shared by the top-k kernel and the fused decode select kernel.
//
// Indexer.forward keeps index_score.topk(...) per query row; the NKI indexer page
// returns the selection as an unordered int32 set.  Here each row's valid prefix
// [0, L) is selected exactly: the min(k, L) largest scores, ties to the lower index,
// -0 equal to +0, unused slots -1.
//
// One block per row, NT = 1024 threads, or 256 when T <= 4096 (short rows then keep
// 16 scores per thread instead of leaving most of a large block idle).  The row is
// read once (from HBM in the top-k kernel, from LDS in the fused decode select) and
// stays in registers: thread t holds elements 4(t + NT j) + c (j, c < 4).
//
// 1. A block reduction finds the row's smallest and largest valid score, lo and hi.
// 2. Each element goes to one of B = 4 NT equal-width bins of [lo, hi] (4096 or 1024):
//    bin(v) + 1 = trunc(fma(v - lo, (B - 1) * rcp(hi - lo), 1)), 1 .. B.  A rounded
//    subtraction, a correctly rounded fma with a positive factor and truncation are
//    each monotone, so v1 < v2 implies bin(v1) <= bin(v2): every element of a higher
//    bin outranks every element of a lower one.  Unlike digits of the float's bits,
//    equal-width bins spread the scores of a row evenly, so LDS histogram updates
//    rarely collide and the bin that holds the k-th largest score holds few elements.
// 3. A block scan of the histogram from the top finds that bin b and how many of
//    its elements are still needed.
// 4. Inside bin b the exact cut is found: if the bin is taken whole, nothing more;
//    if it holds at most NT / 4 elements, they go to LDS and are ranked pairwise
//    (score descending, index ascending; 4 lanes per element) in step 5; otherwise a
//    radix select walks the 32-bit order-preserving key of the bin's elements with
//    digits of 12, 11 and 9 bits (10, 10, 10 and 2 with 1024 bins).
//    A row whose range is empty or outside [1e-30, 1e30] puts every element in
//    bin 0 and takes the radix path.
// 5. The write-out places the selected elements with one block-wide scan of packed
//    per-thread counts, so the result is deterministic: an upper group (the higher
//    bins, and after a radix cut the part of the cut bin above the cut) in increasing
//    index order, then the cut group: after a pairwise cut its `need` best elements in
//    rank order (score descending, index ascending), each stored by the lanes that
//    ranked it; otherwise the taken elements at the cut in increasing index order
//    (lowest indices first).  Every score of the upper group is at least every score
//    of the cut group (strictly above after a radix cut or a bin taken whole).
//
// Wave-level scans and reductions use DPP row shifts and row broadcasts; a reduction
// over the 16 waves' partial results uses one DPP row.
#pragma once
#include "lk_device.h"

namespace lk {
namespace {

// Block shapes: NT threads (1024, or 256 for rows of at most 4096 scores), 16 scores
// per thread, 4 histogram bins per thread.
constexpr int kPer = 16;                    // elements per thread
template <int NT>
struct Shape {
    static constexpr int kThreads = NT, kWaves = NT / 64, kBins = 4 * NT, kMaxT = NT * kPer;
    // A cut bin of at most kSmall elements is ranked pairwise, kLanesPerCand lanes per
    // candidate (each comparing every kLanesPerCand-th group of 4 candidates).
    static constexpr int kSmall = NT / 4, kLanesPerCand = NT / kSmall;
    static_assert(kWaves >= 4 && kWaves <= 16 && (kWaves & (kWaves - 1)) == 0, "one DPP row holds the wave totals");
    static_assert(kSmall % 4 == 0 && (kLanesPerCand & (kLanesPerCand - 1)) == 0 && kLanesPerCand <= 4,
                  "16-byte candidate reads; a candidate's lanes sit in one DPP quad");
};

// Larger float -> larger key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over the 64 lanes of a wave (DPP: row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Inclusive scan within each 16-lane DPP row; lane 16r + 15 ends with row r's sum.
__device__ __forceinline__ uint32_t row_scan16(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    return x;
}

// Running maximum and minimum over lanes with one DPP-routed v_max_f32 / v_min_f32 per
// step.  A lane whose source is outside its row, or whose row is masked off, is not
// written and keeps its value; a quiet-NaN operand yields the other operand (IEEE
// mode), as fmaxf / fminf do.  The leading s_nop gives the DPP read of a VGPR written
// by the previous VALU instruction its two wait states.
#define LK_DPP_STEP(op, x, ctrl) asm("s_nop 1\n\t" op "_dpp %0, %0, %0 " ctrl : "+v"(x))
// Lane 16r + 15 ends with the result over DPP row r.
__device__ __forceinline__ float row_fmax16(float x) {
    LK_DPP_STEP("v_max_f32", x, "row_shr:1 row_mask:0xf bank_mask:0xf");
    LK_DPP_STEP("v_max_f32", x, "row_shr:2 row_mask:0xf bank_mask:0xf");
    LK_DPP_STEP("v_max_f32", x, "row_shr:4 row_mask:0xf bank_mask:0xf");
    LK_DPP_STEP("v_max_f32", x, "row_shr:8 row_mask:0xf bank_mask:0xf");
    return x;
}
__device__ __forceinline__ float row_fmin16(float x) {
    LK_DPP_STEP("v_min_f32", x, "row_shr:1 row_mask:0xf bank_mask:0xf");
    LK_DPP_STEP("v_min_f32", x, "row_shr:2 row_mask:0xf bank_mask:0xf");
    LK_DPP_STEP("v_min_f32", x, "row_shr:4 row_mask:0xf bank_mask:0xf");
    LK_DPP_STEP("v_min_f32", x, "row_shr:8 row_mask:0xf bank_mask:0xf");
    return x;
}
// Lane 63 ends with the result over the wave.
__device__ __forceinline__ float wave_fmax(float x) {
    x = row_fmax16(x);
    LK_DPP_STEP("v_max_f32", x, "row_bcast:15 row_mask:0xa bank_mask:0xf");
    LK_DPP_STEP("v_max_f32", x, "row_bcast:31 row_mask:0xc bank_mask:0xf");
    return x;
}
__device__ __forceinline__ float wave_fmin(float x) {
    x = row_fmin16(x);
    LK_DPP_STEP("v_min_f32", x, "row_bcast:15 row_mask:0xa bank_mask:0xf");
    LK_DPP_STEP("v_min_f32", x, "row_bcast:31 row_mask:0xc bank_mask:0xf");
    return x;
}
#undef LK_DPP_STEP

// Sum of the per-wave totals of waves 0 .. wave-1 (before) and of all kWaves waves
// (total), computed by every wave from the kWaves words of `part` (one per wave).
template <int kWaves>
__device__ __forceinline__ void wave_prefix(const uint32_t *part, int wave, uint32_t &before, uint32_t &total) {
    const int lane = __lane_id();
    const uint32_t s = row_scan16(lane < kWaves ? part[lane] : 0u);   // DPP row 0 holds them all
    total = (uint32_t)__builtin_amdgcn_readlane((int)s, kWaves - 1);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)s, (wave + kWaves - 1) & (kWaves - 1));
    before = wave > 0 ? b : 0u;
}

// Block-wide selection: the bin holding the need-th largest counted element (counting
// from the top bin) and the number of counted elements in higher bins; writes
// (bin, above, count) to sel.  Thread t owns bins kBins-1-4t .. kBins-4-4t (one
// 16-byte read), scans within its wave with DPP and across waves through wsum.  Ends
// with a barrier after which sel is valid.
template <int NT>
__device__ __forceinline__ void select_bin(const uint32_t *hist, uint32_t need, uint32_t *wsum, uint32_t *sel,
                                           int tid) {
    const int lane = __lane_id(), wave = tid >> 6;
    const int lo = Shape<NT>::kBins - 4 - 4 * tid;     // bins lo .. lo+3, owned top-down
    const uint4 h = *reinterpret_cast<const uint4 *>(hist + lo);
    const uint32_t mine = h.x + h.y + h.z + h.w;
    const uint32_t incl = wave_scan(mine);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before, total;
    wave_prefix<Shape<NT>::kWaves>(wsum, wave, before, total);
    uint32_t above = before + incl - mine;
    const uint32_t c[4] = {h.w, h.z, h.y, h.x};        // c[q] = bin lo+3-q
#pragma unroll
    for (int q = 0; q < 4; q++) {
        if (above < need && above + c[q] >= need) {
            sel[0] = (uint32_t)(lo + 3 - q);
            sel[1] = above;
            sel[2] = c[q];
        }
        above += c[q];
    }
    __syncthreads();
}

__device__ __forceinline__ void clear_hist(uint32_t *hist, int tid) {
    reinterpret_cast<uint4 *>(hist)[tid] = make_uint4(0, 0, 0, 0);   // 4 bins per thread
}

// Index of element e of thread tid.
template <int NT>
__device__ __forceinline__ uint32_t elem_index(int tid, int e) {
    return 4u * tid + 4u * NT * (e >> 2) + (e & 3);
}

// The block's LDS for one row, as pointers to wherever the calling kernel keeps it.
template <int NT>
struct TopkLds {
    uint32_t *hist_buf;                         // 4 + Shape<NT>::kBins words, 16-byte aligned; word 3: invalid elements
    uint32_t (*wtot)[4];                        // [kWaves][4], 16-byte aligned
    uint32_t *wsum;                             // [kWaves]
    float (*wred)[Shape<NT>::kWaves];           // [2][kWaves]
    uint32_t *sel;                              // [3]
    uint32_t *cand_key;                         // [kSmall], 16-byte aligned
    uint32_t *cand_idx;                         // [kSmall], 16-byte aligned
    uint32_t *ccount;
};

// The same LDS as one object, for a kernel that holds it in a struct.
template <int NT>
struct TopkShared {
    uint32_t hist_buf[4 + Shape<NT>::kBins] __attribute__((aligned(16)));
    uint32_t wtot[Shape<NT>::kWaves][4] __attribute__((aligned(16)));
    uint32_t wsum[Shape<NT>::kWaves];
    float wred[2][Shape<NT>::kWaves];
    uint32_t sel[3];
    uint32_t cand_key[Shape<NT>::kSmall] __attribute__((aligned(16)));
    uint32_t cand_idx[Shape<NT>::kSmall] __attribute__((aligned(16)));
    uint32_t ccount;
    __device__ TopkLds<NT> view() { return {hist_buf, wtot, wsum, wred, sel, cand_key, cand_idx, &ccount}; }
};

// The top-k of one row: the min(k, L) largest of src[0 .. L-1] into out[0 .. k-1] (-1
// after them), computed by the NT threads tid = 0 .. NT-1 of the calling block, which
// all call it; every other wave of the block has ended (the barriers inside count only
// waves still running).  src holds T readable floats (T >= L); requires 1 <= k and
// L <= Shape<NT>::kMaxT.
template <int NT>
__device__ __forceinline__ void topk_row(const float *src, int64_t T, int64_t L, int32_t k,
                                         int32_t *out, int tid, const TopkLds<NT> &sh) {
    constexpr int kThreads = Shape<NT>::kThreads, kWaves = Shape<NT>::kWaves, kBins = Shape<NT>::kBins;
    constexpr int kSmall = Shape<NT>::kSmall, kLanesPerCand = Shape<NT>::kLanesPerCand;
    uint32_t *const hist = sh.hist_buf + 4;            // bins 0 .. kBins-1
    uint32_t (*const wtot)[4] = sh.wtot;
    uint32_t *const wsum = sh.wsum;
    float (*const wred)[kWaves] = sh.wred;
    uint32_t *const sel = sh.sel;
    uint32_t *const cand_key = sh.cand_key;
    uint32_t *const cand_idx = sh.cand_idx;
    uint32_t &ccount = *sh.ccount;
    const int lane = __lane_id(), wave = tid >> 6;
    if (L <= k) {                                      // everything valid is selected
        for (int64_t j = tid; j < k; j += kThreads) out[j] = j < L ? (int32_t)j : -1;
        return;
    }
    const int n = (int)L;                              // k < L <= Shape<NT>::kMaxT (caller's choice)

    clear_hist(hist, tid);
    if (tid == 0) ccount = 0;
    // Element e of this thread has index elem_index(tid, e); elements past the valid
    // prefix hold NaN.  Group j (elements 4j..4j+3) of a wave is `live` when it holds
    // at least one valid element; a dead group is skipped by every later pass.
    const float qnan = __int_as_float(0x7FC00000);
    float v[kPer];
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (T & 3) == 0;
    const int rem = n - 4 * tid;                       // element e is valid iff its offset < rem
    const int wave_rem = n - 4 * 64 * wave;            // the same for the wave's first lane
    auto live = [&](int j) { return 4 * kThreads * j < wave_rem; };
    if (vec && rem > 4 * kThreads * 3 + 3) {
        // Every element of this thread is valid: four unconditional loads, all in flight
        // together (under the branches below each one would be waited for alone).
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float4 x = *reinterpret_cast<const float4 *>(src + 4 * tid + 4 * kThreads * j);
            v[4 * j] = x.x; v[4 * j + 1] = x.y; v[4 * j + 2] = x.z; v[4 * j + 3] = x.w;
        }
    } else {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int o = 4 * kThreads * j;
        float4 x = make_float4(qnan, qnan, qnan, qnan);
        if (live(j)) {
            if (vec) {
                // A float4 group that starts below n ends below T (T % 4 == 0): in bounds.
                if (o < rem) x = *reinterpret_cast<const float4 *>(src + 4 * tid + o);
                if (o + 1 >= rem) x.y = qnan;
                if (o + 2 >= rem) x.z = qnan;
                if (o + 3 >= rem) x.w = qnan;
            } else {
                if (o < rem) x.x = src[4 * tid + o];
                if (o + 1 < rem) x.y = src[4 * tid + o + 1];
                if (o + 2 < rem) x.z = src[4 * tid + o + 2];
                if (o + 3 < rem) x.w = src[4 * tid + o + 3];
            }
        }
        v[4 * j] = x.x; v[4 * j + 1] = x.y; v[4 * j + 2] = x.z; v[4 * j + 3] = x.w;
    }
    }

    // 1. Row range (NaN entries are ignored by fmaxf / fminf).
    float mx = v[0], mn = v[0];
#pragma unroll
    for (int e = 1; e < kPer; e++) {
        mx = fmaxf(mx, v[e]);
        mn = fminf(mn, v[e]);
    }
    mx = wave_fmax(mx);
    mn = wave_fmin(mn);
    if (lane == 63) {
        wred[0][wave] = mx;
        wred[1][wave] = mn;
    }
    __syncthreads();
    // Every wave reduces the kWaves partial results itself (lane l reads wave
    // l % kWaves, so one DPP row holds all of them).
    mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row_fmax16(wred[0][lane & (kWaves - 1)])), 15));
    mn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row_fmin16(wred[1][lane & (kWaves - 1)])), 15));
    const float width = mx - mn;
    const bool spread = width >= 1e-30f && width <= 1e30f;
    // scale = (kBins - 1) * rcp(width), the hardware reciprocal (within 1 ulp), keeps
    // fma(v - mn, scale, 1) below kBins + 1, and every valid score of a spread row is
    // finite, so bin + 1 is 1 .. kBins; it is monotone in v (a rounded subtraction,
    // then a correctly rounded fma with a positive factor, then truncation).
    const float scale = (float)(kBins - 1) * __builtin_amdgcn_rcpf(width);

    // 2-3. Histogram of the bins (invalid elements count in hist[-1], a spare word),
    //      then the bin holding the k-th largest.
    // bin + 1 of every element is kept in 16-bit halves for the classification below;
    // an invalid element (NaN) and every element of a dead group keep 0.  A wave whose
    // elements are all valid takes a straight-line loop without those checks.
    uint32_t bins[kPer / 2] = {};
    const bool wave_full = wave_rem >= 4 * kThreads * (kPer / 4 - 1) + 4 * 64;
    if (spread && wave_full) {
#pragma unroll
        for (int e = 0; e < kPer; e++) {
            const uint32_t b1 = (uint32_t)fmaf(v[e] - mn, scale, 1.0f);
            bins[e >> 1] |= b1 << (16 * (e & 1));
            atomicAdd(&hist[(int)b1 - 1], 1u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kPer; e++) {
            if (!live(e >> 2)) continue;
            // fmaxf maps NaN to 0; a row without spread puts every valid element in bin 0.
            const int b1 = spread ? (int)fmaxf(fmaf(v[e] - mn, scale, 1.0f), 0.0f) : (v[e] == v[e] ? 1 : 0);
            bins[e >> 1] |= (uint32_t)b1 << (16 * (e & 1));
            atomicAdd(&hist[b1 - 1], 1u);
        }
    }
    __syncthreads();
    select_bin<NT>(hist, (uint32_t)k, wsum, sel, tid);
    const uint32_t cb = sel[0], cnt = sel[2];
    uint32_t need = (uint32_t)k - sel[1];

    // 4. Classify: gbits = elements of higher bins (taken), ebits = elements of bin cb.
    //    An invalid or dead element (bin + 1 == 0) is in neither.
    uint32_t gbits = 0, ebits = 0;
#pragma unroll
    for (int e = 0; e < kPer; e++) {
        const uint32_t b1 = (bins[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        gbits |= (b1 > cb + 1 ? 1u : 0u) << e;
        ebits |= (b1 == cb + 1 ? 1u : 0u) << e;
    }
    // The cut inside bin cb.  A bin taken whole needs none.  A small bin is ranked
    // pairwise after the write-out barrier (below); its elements leave ebits.  A larger
    // one is cut by a radix select: of its elements, those whose key & pmask exceeds
    // prefix join gbits, and the `need` lowest-index ones whose key & pmask equals
    // prefix stay in ebits.
    const bool pairwise = need < cnt && cnt <= (uint32_t)kSmall;
    uint32_t prefix = 0, pmask = 0;
    if (pairwise) {
        for (uint32_t m = ebits; m; m &= m - 1) {
            const int e = __builtin_ctz(m);
            const uint32_t slot = atomicAdd(&ccount, 1u);
            cand_key[slot] = order_key(v[e]);
            cand_idx[slot] = elem_index<NT>(tid, e);
        }
        ebits = 0;
    } else if (need < cnt) {
        // Digits of at most log2(kBins) bits from the top: key bits 31-20, 19-9, 8-0 with
        // 4096 bins; 31-22, 21-12, 11-2, 1-0 with 1024.
        constexpr int kPasses = kBins == 4096 ? 3 : 4;
        static_assert(kBins == 4096 || kBins == 1024, "digit plan");
#pragma unroll 1
        for (int pass = 0; pass < kPasses; pass++) {
            clear_hist(hist, tid);
            __syncthreads();
            const int sh = kBins == 4096 ? (pass == 0 ? 20 : pass == 1 ? 9 : 0) : (pass == 3 ? 0 : 22 - 10 * pass);
            const uint32_t dm = kBins == 4096 ? (pass == 0 ? 0xFFFu : pass == 1 ? 0x7FFu : 0x1FFu) : (pass == 3 ? 0x3u : 0x3FFu);
            for (uint32_t m = ebits; m; m &= m - 1) {
                const uint32_t kk = order_key(v[__builtin_ctz(m)]);
                if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> sh) & dm], 1u);
            }
            __syncthreads();
            select_bin<NT>(hist, need, wsum, sel, tid);
            const uint32_t d = sel[0], ab = sel[1], dcnt = sel[2];
            need -= ab;
            prefix |= d << sh;
            pmask |= dm << sh;
            if (need == dcnt) break;                   // the whole digit bin is taken (or the key is exact)
        }
        for (uint32_t m = ebits; m; m &= m - 1) {
            const int e = __builtin_ctz(m);
            const uint32_t km = order_key(v[e]) & pmask;
            if (km != prefix) ebits &= ~(1u << e);
            if (km > prefix) gbits |= 1u << e;
        }
    }

    // 5. Write-out.  The upper group (gbits) takes positions 0 .. n_gt - 1 in index
    //    order; the cut group takes n_gt .. k - 1: in index order from ebits (a bin taken
    //    whole, or the radix cut), or, for a pairwise cut, in rank order.
    const uint32_t n_gt = (uint32_t)k - need;
    // Per-row-j counts in 16-bit fields: word 0 = rows 0,1 of gbits; 1 = rows 2,3;
    // words 2, 3 the same for ebits.
    uint32_t cnt4[4];
#pragma unroll
    for (int f = 0; f < 4; f++) {
        const uint32_t bits = (f < 2 ? gbits : ebits) >> (8 * (f & 1));
        cnt4[f] = __builtin_popcount(bits & 0xFu) | (__builtin_popcount((bits >> 4) & 0xFu) << 16);
    }
    uint32_t incl[4];
#pragma unroll
    for (int f = 0; f < 4; f++) incl[f] = wave_scan(cnt4[f]);
    if (lane == 63) *reinterpret_cast<uint4 *>(wtot[wave]) = make_uint4(incl[0], incl[1], incl[2], incl[3]);
    __syncthreads();                                   // also publishes the pairwise candidates
    char *const outb = reinterpret_cast<char *>(out);
    if (pairwise) {
        // Rank of candidate ci = tid / kLanesPerCand among the cnt candidates (score
        // descending, index ascending): its lanes each compare it with every
        // kLanesPerCand-th group of 4 candidates and sum packed counts (above: low half,
        // equal with a lower index: high half); the last of them stores it at n_gt + rank
        // when the rank is below `need`.  Ranks are distinct, so each position of the
        // cut group is written once.
        const int ci = tid / kLanesPerCand, q = tid % kLanesPerCand;
        uint32_t packed = 0, mk = 0, mi = 0;
        if (ci < (int)cnt) {
            mk = cand_key[ci];
            mi = cand_idx[ci];
            for (int g = q; 4 * g < (int)cnt; g += kLanesPerCand) {
                const uint4 kq = *reinterpret_cast<const uint4 *>(cand_key + 4 * g);
                const uint4 iq = *reinterpret_cast<const uint4 *>(cand_idx + 4 * g);
                const uint32_t kj[4] = {kq.x, kq.y, kq.z, kq.w}, ij[4] = {iq.x, iq.y, iq.z, iq.w};
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    if (4 * g + jj < (int)cnt) {
                        packed += kj[jj] > mk ? 1u : 0u;
                        packed += (kj[jj] == mk && ij[jj] < mi) ? 0x10000u : 0u;
                    }
                }
            }
        }
#pragma unroll
        for (int d = 1; d < kLanesPerCand; d <<= 1) packed += (uint32_t)__shfl_xor((int)packed, d, 64);
        const uint32_t rank = (packed & 0xFFFFu) + (packed >> 16);
        if (q == kLanesPerCand - 1 && ci < (int)cnt && rank < need)
            *reinterpret_cast<int32_t *>(outb + 4u * (n_gt + rank)) = (int32_t)mi;
    }
    // The four fields' sums over the lower waves and over all waves: lane l < 16 reads
    // wave l's totals (DPP row 0 holds them all) and the four row scans run together.
    uint32_t before[4], total[4];
    {
        const uint4 wt = lane < kWaves ? *reinterpret_cast<const uint4 *>(wtot[lane]) : make_uint4(0, 0, 0, 0);
        const uint32_t sc[4] = {row_scan16(wt.x), row_scan16(wt.y), row_scan16(wt.z), row_scan16(wt.w)};
#pragma unroll
        for (int f = 0; f < 4; f++) {
            total[f] = (uint32_t)__builtin_amdgcn_readlane((int)sc[f], kWaves - 1);
            const uint32_t bf = (uint32_t)__builtin_amdgcn_readlane((int)sc[f], (wave + kWaves - 1) & (kWaves - 1));
            before[f] = wave > 0 ? bf : 0u;
        }
    }
    // Stores address the row by 32-bit byte offsets (positions kept times 4).  The upper
    // group holds exactly n_gt elements (every element above the cut, counted by the
    // selection), so its offsets stay below 4 n_gt; the clamp to the row only keeps a
    // store in bounds should that ever fail.
    const uint32_t row_end4 = 4u * (uint32_t)(k - 1);
    uint32_t gbase = 0, ebase = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t gx = incl[h] - cnt4[h] + before[h], ex = incl[2 + h] - cnt4[2 + h] + before[2 + h];
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const int j = 2 * h + half;
            const int32_t base = 4 * (tid + kThreads * j);
            uint32_t gm = (gbits >> (4 * j)) & 0xFu, em = (ebits >> (4 * j)) & 0xFu;
            uint32_t g4 = 4u * (gbase + ((gx >> (16 * half)) & 0xFFFFu));
            uint32_t er = ebase + ((ex >> (16 * half)) & 0xFFFFu);
            while (gm) {
                const int c = __builtin_ctz(gm);
                gm &= gm - 1;
                *reinterpret_cast<int32_t *>(outb + min(g4, row_end4)) = base + c;
                g4 += 4u;
            }
            while (em) {
                const int c = __builtin_ctz(em);
                em &= em - 1;
                if (er < need) *reinterpret_cast<int32_t *>(outb + 4u * (n_gt + er)) = base + c;
                er++;
            }
            gbase += (total[h] >> (16 * half)) & 0xFFFFu;
            ebase += (total[2 + h] >> (16 * half)) & 0xFFFFu;
        }
    }
}

}  // namespace
}  // namespace lk

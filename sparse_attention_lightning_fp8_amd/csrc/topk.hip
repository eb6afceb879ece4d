// topk.hip -- per-row top-k of the index scores (gfx950).
//
// Indexer.forward keeps index_score.topk(...) per query row; the NKI indexer page
// returns the selection as an unordered int32 set.  Here each row's valid prefix
// [0, L) is selected exactly: the min(k, L) largest scores, ties to the lower index,
// -0 equal to +0, unused slots -1.
//
// One block of 1024 threads per row.  The row is read from HBM once and stays in
// registers: thread t holds elements 4(t + 1024 j) + c (j, c < 4) as order-preserving
// 32-bit keys.  A radix select walks the key from the top with digits of 12, 11 and
// 9 bits; each pass histograms (in LDS) the next digit of the elements that still
// match the chosen prefix, and a block scan picks the bin holding the k-th largest.  As
// soon as the chosen bin is taken whole, the remaining digits cannot change the
// selected set and the walk stops (the common case after two passes).  The write-out
// ranks the selected elements with one block-wide scan of packed per-thread counts, so
// the result is deterministic: every index whose key is above the final prefix in
// increasing order, then the lowest-index elements equal to it.
//
// The histogram has four copies (lane & 3 picks one; copies are padded onto different
// banks) so that lanes of one wave that hit the same bin mostly update different
// words.  Wave-level scans use DPP row shifts and row broadcasts.
#include "lk_device.h"

namespace lk {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 16;                    // elements per thread (kThreads * kPer == LK_TOPK_MAX_T)
constexpr int kBins = 4096;
constexpr int kCopies = 4;
constexpr int kCopyStride = kBins + 4;      // +4 words: copies start on different banks, 16-B aligned

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

// Block-wide selection: the bin holding the need-th largest counted element (counting
// from the top bin) and the number of counted elements in higher bins; writes
// (bin, above, count) to sel.  Thread t owns bins 4095-4t .. 4092-4t (one 16-byte read
// per histogram copy, conflict-free), scans within its wave with DPP and across waves
// through wsum.  Ends with a barrier after which sel is valid.
__device__ __forceinline__ void select_bin(const uint32_t *hist, uint32_t need, uint32_t *wsum, uint32_t *sel) {
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
    const int lo = kBins - 4 - 4 * tid;                // bins lo .. lo+3, owned top-down
    uint32_t c[4] = {0, 0, 0, 0};
#pragma unroll
    for (int cp = 0; cp < kCopies; cp++) {
        const uint32_t *h = hist + cp * kCopyStride + lo;
#pragma unroll
        for (int q = 0; q < 4; q++) c[q] += h[3 - q];  // c[q] = bin lo+3-q
    }
    const uint32_t mine = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_scan(mine);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t above = incl - mine;
    for (int w = 0; w < wave; w++) above += wsum[w];
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

__global__ void __launch_bounds__(kThreads)
topk_kernel(const float *__restrict__ scores, RowsDev rows, int32_t k, int32_t *__restrict__ idx) {
    __shared__ __attribute__((aligned(16))) uint32_t hist[kCopies * kCopyStride + 3];
    __shared__ uint32_t wtot[kWaves][4];
    __shared__ uint32_t wsum[kWaves];
    __shared__ uint32_t sel[3];

    const int row = blockIdx.x;
    const int b = row / rows.S;
    const int t = row - b * rows.S;
    const int64_t T = rows.T;
    const int64_t L = row_len(rows, b, t);
    int32_t *out = idx + (int64_t)row * k;
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
    if (L <= k) {                                      // everything valid is selected
        for (int64_t j = tid; j < k; j += kThreads) out[j] = j < L ? (int32_t)j : -1;
        return;
    }
    const int n = (int)L;                              // k < L <= T <= LK_TOPK_MAX_T
    const float *src = scores + (int64_t)row * T;

    for (int i = tid; i < kCopies * kCopyStride; i += kThreads) hist[i] = 0;
    // Element (j, c) of this thread is index 4 (tid + 1024 j) + c.
    uint32_t key[kPer];
    uint32_t valid = 0;                                // bit 4j + c
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int i0 = 4 * (tid + kThreads * j);
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (vec && i0 + 3 < n) {
            const float4 x = *reinterpret_cast<const float4 *>(src + i0);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++)
                if (i0 + c < n) v[c] = src[i0 + c];
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            key[4 * j + c] = order_key(v[c]);
            if (i0 + c < n) valid |= 1u << (4 * j + c);
        }
    }
    uint32_t *my_hist = hist + (lane & (kCopies - 1)) * kCopyStride;
    __syncthreads();

    // Radix select from the top: digits of 12, 11 and 9 bits.
    uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
    const int shifts[3] = {20, 9, 0};
    const uint32_t dmasks[3] = {0xFFFu, 0x7FFu, 0x1FFu};
#pragma unroll 1
    for (int pass = 0; pass < 3; pass++) {
        const int sh = shifts[pass];
        const uint32_t dm = dmasks[pass];
#pragma unroll
        for (int e = 0; e < kPer; e++)
            if (((valid >> e) & 1u) && (key[e] & pmask) == prefix) atomicAdd(&my_hist[(key[e] >> sh) & dm], 1u);
        __syncthreads();
        select_bin(hist, need, wsum, sel);
        const uint32_t d = sel[0], ab = sel[1], cnt = sel[2];
        need -= ab;
        prefix |= d << sh;
        pmask |= dm << sh;
        if (need == cnt || pass == 2) break;           // the whole bin is taken (or K* is exact)
        for (int i = tid; i < kCopies * kCopyStride; i += kThreads) hist[i] = 0;
        __syncthreads();
    }
    // Selected: (key & pmask) > prefix  (n_gt of them), and the `need` lowest-index
    // elements with (key & pmask) == prefix.
    const uint32_t n_gt = (uint32_t)k - need;
    uint32_t gbits = 0, ebits = 0;
#pragma unroll
    for (int e = 0; e < kPer; e++) {
        const uint32_t m = key[e] & pmask;
        if ((valid >> e) & 1u) {
            gbits |= (m > prefix ? 1u : 0u) << e;
            ebits |= (m == prefix ? 1u : 0u) << e;
        }
    }
    // Per-row-j counts in 16-bit fields: g01 = rows 0,1 of gbits; g23 = rows 2,3; same for e.
    uint32_t cnt4[4];
    {
        const uint32_t g0 = __builtin_popcount(gbits & 0xFu), g1 = __builtin_popcount((gbits >> 4) & 0xFu);
        const uint32_t g2 = __builtin_popcount((gbits >> 8) & 0xFu), g3 = __builtin_popcount((gbits >> 12) & 0xFu);
        const uint32_t e0 = __builtin_popcount(ebits & 0xFu), e1 = __builtin_popcount((ebits >> 4) & 0xFu);
        const uint32_t e2 = __builtin_popcount((ebits >> 8) & 0xFu), e3 = __builtin_popcount((ebits >> 12) & 0xFu);
        cnt4[0] = g0 | (g1 << 16);
        cnt4[1] = g2 | (g3 << 16);
        cnt4[2] = e0 | (e1 << 16);
        cnt4[3] = e2 | (e3 << 16);
    }
    uint32_t incl[4];
#pragma unroll
    for (int f = 0; f < 4; f++) incl[f] = wave_scan(cnt4[f]);
    if (lane == 63) {
#pragma unroll
        for (int f = 0; f < 4; f++) wtot[wave][f] = incl[f];
    }
    __syncthreads();
    uint32_t before[4] = {0, 0, 0, 0}, total[4] = {0, 0, 0, 0};
    for (int w = 0; w < kWaves; w++) {
#pragma unroll
        for (int f = 0; f < 4; f++) {
            const uint32_t x = wtot[w][f];
            before[f] += w < wave ? x : 0u;
            total[f] += x;
        }
    }
    // Exclusive prefix per row j for "greater" (fields of words 0,1) and "equal" (2,3).
    uint32_t gpre[4], epre[4], gtot[4], etot[4];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t gx = incl[h] - cnt4[h] + before[h], ex = incl[2 + h] - cnt4[2 + h] + before[2 + h];
        gpre[2 * h] = gx & 0xFFFFu;
        gpre[2 * h + 1] = gx >> 16;
        epre[2 * h] = ex & 0xFFFFu;
        epre[2 * h + 1] = ex >> 16;
        gtot[2 * h] = total[h] & 0xFFFFu;
        gtot[2 * h + 1] = total[h] >> 16;
        etot[2 * h] = total[2 + h] & 0xFFFFu;
        etot[2 * h + 1] = total[2 + h] >> 16;
    }
    uint32_t gbase = 0, ebase = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint32_t gm = (gbits >> (4 * j)) & 0xFu, em = (ebits >> (4 * j)) & 0xFu;
        uint32_t gr = gbase + gpre[j], er = ebase + epre[j];
        while (gm) {
            const int c = __builtin_ctz(gm);
            gm &= gm - 1;
            if (gr < n_gt) out[gr] = 4 * (tid + kThreads * j) + c;
            gr++;
        }
        while (em) {
            const int c = __builtin_ctz(em);
            em &= em - 1;
            if (er < need) out[n_gt + er] = 4 * (tid + kThreads * j) + c;
            er++;
        }
        gbase += gtot[j];
        ebase += etot[j];
    }
}

}  // namespace

hipError_t launch_topk(const float *scores, const RowsDev &rows, int32_t k, int32_t *idx, hipStream_t stream) {
    const unsigned nrows = (unsigned)((int64_t)rows.B * rows.S);
    return launch(topk_kernel, dim3(nrows), dim3(kThreads), 0u, stream, scores, rows, k, idx);
}

}  // namespace lk

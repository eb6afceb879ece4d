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
// match the chosen prefix, and picks the bin holding the k-th largest.  As soon as
// the chosen bin is taken whole, the remaining digits cannot change the selected set
// and the walk stops early (the common case after two passes).  The write-out ranks
// the selected elements with one block-wide scan of packed per-thread counts, so the
// result is deterministic: every index whose key is above the final prefix in
// increasing order, then the lowest-index elements equal to it.
#include "lk_device.h"

namespace lk {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 16;                    // elements per thread (kThreads * kPer == LK_TOPK_MAX_T)
constexpr int kBins = 4096;

// Larger float -> larger key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive scan of two packed uint64 values (tmp: 2 * kWaves entries).
// Returns the exclusive prefixes and the block totals.
__device__ __forceinline__ void block_scan2(uint64_t a, uint64_t b, uint64_t *tmp, uint64_t &pa, uint64_t &pb,
                                            uint64_t &ta, uint64_t &tb) {
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
    uint64_t va = a, vb = b;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t ya = __shfl_up(va, d, 64), yb = __shfl_up(vb, d, 64);
        if (lane >= d) {
            va += ya;
            vb += yb;
        }
    }
    if (lane == 63) {
        tmp[wave] = va;
        tmp[kWaves + wave] = vb;
    }
    __syncthreads();
    uint64_t ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        const uint64_t xa = tmp[w], xb = tmp[kWaves + w];
        ba += w < wave ? xa : 0;
        bb += w < wave ? xb : 0;
        sa += xa;
        sb += xb;
    }
    __syncthreads();
    pa = va - a + ba;
    pb = vb - b + bb;
    ta = sa;
    tb = sb;
}

// Inclusive block scan of one uint32 per thread (tmp: kWaves entries).
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *tmp) {
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(v, d, 64);
        if (lane >= d) v += y;
    }
    if (lane == 63) tmp[wave] = v;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) before += w < wave ? tmp[w] : 0u;
    __syncthreads();
    return v + before;
}

__global__ void __launch_bounds__(kThreads)
topk_kernel(const float *__restrict__ scores, RowsDev rows, int32_t k, int32_t *__restrict__ idx) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint64_t scan64[2 * kWaves];
    __shared__ uint32_t scan32[kWaves];
    __shared__ uint32_t sel[3];

    const int row = blockIdx.x;
    const int b = row / rows.S;
    const int t = row - b * rows.S;
    const int64_t T = rows.T;
    const int64_t L = row_len(rows, b, t);
    int32_t *out = idx + (int64_t)row * k;
    const int tid = threadIdx.x;
    if (L <= k) {                                      // everything valid is selected
        for (int64_t j = tid; j < k; j += kThreads) out[j] = j < L ? (int32_t)j : -1;
        return;
    }
    const int n = (int)L;                              // k < L <= T <= LK_TOPK_MAX_T
    const float *src = scores + (int64_t)row * T;

    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
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
            if (((valid >> e) & 1u) && (key[e] & pmask) == prefix) atomicAdd(&hist[(key[e] >> sh) & dm], 1u);
        __syncthreads();
        // Suffix sums from the top bin: thread owns bins 4095-4tid .. 4092-4tid.
        const int top = kBins - 1 - 4 * tid;
        uint32_t c[4];
#pragma unroll
        for (int q = 0; q < 4; q++) c[q] = hist[top - q];
        const uint32_t mine = c[0] + c[1] + c[2] + c[3];
        uint32_t above = block_scan(mine, scan32) - mine;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            if (above < need && above + c[q] >= need) {
                sel[0] = (uint32_t)(top - q);
                sel[1] = above;
                sel[2] = c[q];
            }
            above += c[q];
        }
        __syncthreads();
        const uint32_t d = sel[0], ab = sel[1], cnt = sel[2];
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
        need -= ab;
        prefix |= d << sh;
        pmask |= dm << sh;
        __syncthreads();
        if (need == cnt) break;                        // the whole bin is taken: the set is fixed
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
    uint64_t gpack = 0, epack = 0;                     // per-row-j counts in 16-bit fields
#pragma unroll
    for (int j = 0; j < 4; j++) {
        gpack |= (uint64_t)__builtin_popcount((gbits >> (4 * j)) & 0xFu) << (16 * j);
        epack |= (uint64_t)__builtin_popcount((ebits >> (4 * j)) & 0xFu) << (16 * j);
    }
    uint64_t gpre, epre, gtot, etot;
    block_scan2(gpack, epack, scan64, gpre, epre, gtot, etot);
    uint32_t gbase = 0, ebase = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint32_t gr = gbase + (uint32_t)((gpre >> (16 * j)) & 0xFFFFu);
        uint32_t er = ebase + (uint32_t)((epre >> (16 * j)) & 0xFFFFu);
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int e = 4 * j + c;
            const int i = 4 * (tid + kThreads * j) + c;
            if ((gbits >> e) & 1u) {
                if (gr < n_gt) out[gr] = i;
                gr++;
            }
            if ((ebits >> e) & 1u) {
                if (er < need) out[n_gt + er] = i;
                er++;
            }
        }
        gbase += (uint32_t)((gtot >> (16 * j)) & 0xFFFFu);
        ebase += (uint32_t)((etot >> (16 * j)) & 0xFFFFu);
    }
}

}  // namespace

hipError_t launch_topk(const float *scores, const RowsDev &rows, int32_t k, int32_t *idx, hipStream_t stream) {
    const unsigned nrows = (unsigned)((int64_t)rows.B * rows.S);
    return launch(topk_kernel, dim3(nrows), dim3(kThreads), 0u, stream, scores, rows, k, idx);
}

}  // namespace lk

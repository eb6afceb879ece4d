// topk.hip -- per-row top-k of the index scores (gfx950).
//
// Indexer.forward keeps index_score.topk(...) per query row; the NKI indexer page
// returns the selection as an unordered int32 set.  Here each row's valid prefix
// [0, L) is selected exactly: the min(k, L) largest scores, ties to the lower index,
// -0 equal to +0, unused slots -1.
//
// One block of 1024 threads per row.  The row is loaded once from HBM into LDS as
// order-preserving 32-bit keys; a three-pass radix select (digits of 11, 11 and 10
// bits, MSB first, LDS histograms) finds the exact k-th largest key K*; a final pass
// writes every element above K* and the lowest-index elements equal to K*, in index
// order, using block-wide prefix sums.
#include "lk_device.h"

namespace lk {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

// Larger float -> larger key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the block of one value per thread; `tmp` holds kWaves
// entries.  Returns (inclusive, total).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t *tmp, uint32_t &total) {
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(v, d, 64);
        if (lane >= d) v += y;
    }
    if (lane == 63) tmp[wave] = v;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        const uint32_t x = tmp[w];
        before += w < wave ? x : 0;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return v + before;
}

__global__ void __launch_bounds__(kThreads)
topk_kernel(const float *__restrict__ scores, RowsDev rows, int32_t k, int32_t *__restrict__ idx) {
    __shared__ uint32_t skey[LK_TOPK_MAX_T];
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t scan_tmp[kWaves];
    __shared__ uint32_t sel[2];       // chosen digit, count strictly above it

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
    const int n = (int)L;                              // L <= T <= LK_TOPK_MAX_T
    const float *src = scores + (int64_t)row * T;
    for (int i = tid; i < n; i += kThreads) skey[i] = order_key(src[i]);

    // Radix select: find K* = the k-th largest key.
    uint32_t prefix = 0, prefix_mask = 0;
    int need = k;                                      // how many still to take at/below the prefix
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; pass++) {
        const int sh = shifts[pass];
        const uint32_t dmask = (1u << widths[pass]) - 1u;
        for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint32_t key = skey[i];
            if ((key & prefix_mask) == prefix) atomicAdd(&hist[(key >> sh) & dmask], 1u);
        }
        __syncthreads();
        // Suffix sums from the top bin: each thread owns 2 bins (bins 2047-2tid, 2046-2tid).
        const int hi_bin = kBins - 1 - 2 * tid;
        const uint32_t c_hi = hist[hi_bin], c_lo = hist[hi_bin - 1];
        uint32_t total;
        const uint32_t incl = block_inclusive_scan(c_hi + c_lo, scan_tmp, total);
        const uint32_t above = incl - (c_hi + c_lo);   // count in bins above hi_bin
        // The k-th largest lies in the first bin (from the top) where the running count reaches need.
        if (above < (uint32_t)need && above + c_hi >= (uint32_t)need) {
            sel[0] = (uint32_t)hi_bin;
            sel[1] = above;
        } else if (above + c_hi < (uint32_t)need && above + c_hi + c_lo >= (uint32_t)need) {
            sel[0] = (uint32_t)(hi_bin - 1);
            sel[1] = above + c_hi;
        }
        __syncthreads();
        const uint32_t digit = sel[0];
        need -= (int)sel[1];
        prefix |= digit << sh;
        prefix_mask |= dmask << sh;
        __syncthreads();
    }
    const uint32_t kstar = prefix;                     // exact k-th largest key
    // need = number of elements equal to K* to take (lowest indices first).

    // Final pass: contiguous chunk per thread so index order follows thread order.
    const int chunk = (n + kThreads - 1) / kThreads;
    const int i0 = tid * chunk;
    const int i1 = min(i0 + chunk, n);
    uint32_t gt = 0, eq = 0;
    for (int i = i0; i < i1; i++) {
        const uint32_t key = skey[i];
        gt += key > kstar;
        eq += key == kstar;
    }
    uint32_t gt_total, eq_total;
    const uint32_t gt_pos = block_inclusive_scan(gt, scan_tmp, gt_total) - gt;
    const uint32_t eq_pos = block_inclusive_scan(eq, scan_tmp, eq_total) - eq;
    if (need < 0 || need > k) need = 0;               // unreachable; keeps every write inside the row
    const uint32_t n_gt = (uint32_t)k - (uint32_t)need;  // == gt_total
    uint32_t og = gt_pos, oe = eq_pos;
    for (int i = i0; i < i1; i++) {
        const uint32_t key = skey[i];
        if (key > kstar) {
            if (og < n_gt) out[og] = i;                // og < n_gt always holds; kept as a bound
            og++;
        } else if (key == kstar) {
            if (oe < (uint32_t)need) out[n_gt + oe] = i;
            oe++;
        }
    }
}

}  // namespace

hipError_t launch_topk(const float *scores, const RowsDev &rows, int32_t k, int32_t *idx, hipStream_t stream) {
    const unsigned nrows = (unsigned)((int64_t)rows.B * rows.S);
    hipLaunchKernelGGL(topk_kernel, dim3(nrows), dim3(kThreads), 0, stream, scores, rows, k, idx);
    return hipGetLastError();
}

}  // namespace lk

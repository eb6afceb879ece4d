// topk.hip -- per-row top-k of the index scores (gfx950): one block per row.  The
// algorithm and its ordering guarantees are described in topk_device.h.
#include "topk_device.h"

namespace lk {
namespace {

template <int NT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8, 8)))
topk_kernel(const float *__restrict__ scores, RowsDev rows, int32_t k, int32_t *__restrict__ idx) {
    constexpr int kWaves = Shape<NT>::kWaves;
    __shared__ __attribute__((aligned(16))) uint32_t hist_buf[4 + Shape<NT>::kBins];
    __shared__ __attribute__((aligned(16))) uint32_t wtot[kWaves][4];
    __shared__ uint32_t wsum[kWaves];
    __shared__ float wred[2][kWaves];
    __shared__ uint32_t sel[3];
    __shared__ __attribute__((aligned(16))) uint32_t cand_key[Shape<NT>::kSmall];
    __shared__ __attribute__((aligned(16))) uint32_t cand_idx[Shape<NT>::kSmall];
    __shared__ uint32_t ccount;
    LK_POISON_LDS_OBJS(hist_buf, wtot, wsum, wred, sel, cand_key, cand_idx, ccount);
    const TopkLds<NT> sh{hist_buf, wtot, wsum, wred, sel, cand_key, cand_idx, &ccount};
    const int row = blockIdx.x;
    const int b = row / rows.S;
    const int t = row - b * rows.S;
    const int64_t T = rows.T;
    topk_row<NT>(scores + (int64_t)row * T, T, row_len(rows, b, t), k, idx + (int64_t)row * k, (int)threadIdx.x, sh);
}

}  // namespace

hipError_t launch_topk(const float *scores, const RowsDev &rows, int32_t k, int32_t *idx, hipStream_t stream) {
    const unsigned nrows = (unsigned)((int64_t)rows.B * rows.S);
    if (rows.T <= Shape<256>::kMaxT)
        return launch(topk_kernel<256>, dim3(nrows), dim3(256), 0u, stream, scores, rows, k, idx);
    return launch(topk_kernel<1024>, dim3(nrows), dim3(1024), 0u, stream, scores, rows, k, idx);
}

}  // namespace lk

// probe.hip -- measurement aids outside the indexer computation (gfx950).
//
//  - probe_empty_kernel: the fixed cost of one launch.
//  - probe_read_kernel: a plain streaming read, the bandwidth any kernel that reads a
//    buffer once can expect on this chip.
//  - probe_fp8_score_kernel: the decode index score (page "Index scores") with the
//    contraction on the fp8 MFMA (v_mfma_f32_16x16x32_fp8_fp8) instead of the exactly
//    converted f16 operands the library's score kernels use.  It exists to measure how
//    far the fp8 matrix core's accumulation lands from the exact scores; nothing in the
//    hot path calls it.
#include "lk_device.h"

namespace lk {
namespace {

__global__ void probe_empty_kernel() {}

// Block g reads the g-th contiguous span of the buffer with 16-byte loads, four in
// flight per thread per step, and folds them into one word per wave so the loads stay.
constexpr int kProbeThreads = 256;
__global__ void __launch_bounds__(kProbeThreads)
probe_read_kernel(const uint4 *__restrict__ src, uint64_t n16, uint32_t *__restrict__ sink) {
    const uint64_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t begin = (uint64_t)blockIdx.x * per_block;
    const uint64_t end = begin + per_block < n16 ? begin + per_block : n16;
    uint32_t acc = 0;
    for (uint64_t i = begin + threadIdx.x; i < end; i += 4 * kProbeThreads) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const uint64_t j = i + (uint64_t)u * kProbeThreads;
            v[u] = j < end ? src[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// One wave scores 16 keys of one decode row.  Operand layout of the 16x16x32 fp8 MFMA:
// lane l supplies row l % 16 of A (a head) and column l % 16 of B (a key), bytes
// 8 (l / 16) .. 8 (l / 16) + 7 of each 32-feature K-step; the accumulator of M-tile mt
// holds, in lane l, key l % 16 and heads 16 mt + 4 (l / 16) + i, i < 4.
typedef float probe_f4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256)
probe_fp8_score_kernel(const uint8_t *__restrict__ q_fp8, const float *__restrict__ w_eff,
                       const uint8_t *__restrict__ k_cache, const float *__restrict__ k_scale,
                       int64_t cache_seq_stride, RowsDev rows, float *__restrict__ scores) {
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
    const int b = blockIdx.y;
    const int kr = lane & 15, kg = lane >> 4;
    const int64_t T = rows.T;
    const int64_t L = row_len(rows, b, 0);
    const int64_t s = (int64_t)blockIdx.x * 64 + wave * 16 + kr;
    const uint8_t *krow = k_cache + ((int64_t)b * cache_seq_stride + (s < L ? s : 0)) * LK_DIM;
    const uint8_t *qrow = q_fp8 + (int64_t)b * LK_HEADS * LK_DIM;
    long bk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) bk[ks] = *reinterpret_cast<const long *>(krow + 32 * ks + 8 * kg);
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        probe_f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const long aq = *reinterpret_cast<const long *>(qrow + (16 * mt + kr) * LK_DIM + 32 * ks + 8 * kg);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(aq, bk[ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
            part = __builtin_fmaf(__builtin_fmaxf(acc[i], 0.0f), w_eff[(int64_t)b * LK_HEADS + 16 * mt + 4 * kg + i], part);
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (kg == 0 && s < T)
        scores[(int64_t)b * T + s] = s < L ? part * k_scale[(int64_t)b * cache_seq_stride + s] : -__builtin_inff();
}

}  // namespace

hipError_t launch_probe_empty(int32_t blocks, hipStream_t stream) {
    return launch(probe_empty_kernel, dim3((unsigned)blocks), dim3(64), 0u, stream);
}

hipError_t launch_probe_read(const void *src, uint64_t bytes, uint32_t *sink, int32_t blocks, hipStream_t stream) {
    return launch(probe_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0u, stream,
                  reinterpret_cast<const uint4 *>(src), bytes / 16, sink);
}

hipError_t launch_probe_fp8_score(const uint8_t *q_fp8, const float *w_eff, const uint8_t *k_cache,
                                  const float *k_scale, int64_t cache_seq_stride, const RowsDev &rows, float *scores,
                                  hipStream_t stream) {
    const dim3 grid((unsigned)((rows.T + 63) / 64), (unsigned)rows.B);
    return launch(probe_fp8_score_kernel, grid, dim3(256), 0u, stream, q_fp8, w_eff, k_cache, k_scale,
                  cache_seq_stride, rows, scores);
}

}  // namespace lk

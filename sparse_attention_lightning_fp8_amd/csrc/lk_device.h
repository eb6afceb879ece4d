// lk_device.h -- device-side helpers shared by the gfx950 kernels of liblk.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "lk.h"

namespace lk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Row-validity parameters passed by value to kernels (mirror of lk_rows).
struct RowsDev {
    int32_t B, S;
    int64_t T, start_pos;
    const int32_t *seq_len;
    int32_t causal;
};

// Valid prefix length of score row (b, t): min(T, seq_len[b], start_pos + t + 1).
__device__ __forceinline__ int64_t row_len(const RowsDev &r, int b, int64_t t) {
    int64_t L = r.T;
    if (r.seq_len) {
        int64_t s = r.seq_len[b];
        if (s < L) L = s;
    }
    if (r.causal) {
        int64_t c = r.start_pos + t + 1;
        if (c < L) L = c;
    }
    return L < 0 ? 0 : L;
}

// Four e4m3fn bytes -> four f16 (exact: every e4m3fn value is an f16 normal or zero).
__device__ __forceinline__ void fp8x4_to_f16(uint32_t v, _Float16 *o) {
    half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
    half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true);
    o[0] = lo[0];
    o[1] = lo[1];
    o[2] = hi[0];
    o[3] = hi[1];
}

// Eight e4m3fn bytes (two dwords) -> one f16x8 MFMA operand.
__device__ __forceinline__ half8 fp8x8_to_half8(uint32_t a, uint32_t b) {
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false);
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true);
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true);
    half8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

// ---- LDS DMA (global_load_lds_*): lane l moves 4 or 16 bytes from its own global
// address src into LDS at lds + 4 l or lds + 16 l.  Written as inline asm so that the
// compiler's automatic waits neither count these loads nor make LDS reads wait for
// them (it cannot tell LDS buffers apart); callers wait with s_waitcnt vmcnt before
// reading what they moved.  The LDS base is an input bound to M0, which the compiler
// writes; a DMA needs one wait state after M0 is written, hence the s_nop.
typedef void __attribute__((address_space(3))) *lds_ptr_t;
__device__ __forceinline__ void dma_b128(const void *src, const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}
__device__ __forceinline__ void dma_b32(const void *src, const void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(base) : "memory");
}
// s_waitcnt immediate that waits until at most n vector memory operations of this wave
// are in flight (vmcnt is 6 bits on gfx950; expcnt and lgkmcnt are left alone).
constexpr int vmcnt_imm(int n) { return 0x3F70 | (n & 15) | ((n >> 4) << 14); }

// Sum across the two 32-lane halves of a wave for two values at once:
// returns, in lanes 0-31, x[l] + x[l+32], and in lanes 32-63, y[l-32] + y[l].
__device__ __forceinline__ float halves_sum_pair(float x, float y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Arguments of the two quantization jobs (keys into the cache; queries + weight fold).
struct KeyJobArgs {
    const uint16_t *x = nullptr;
    int64_t n_seq = 0, n_rows = 0, x_seq_stride = 0;
    uint8_t *cache = nullptr;
    float *cache_scale = nullptr;
    int64_t cache_seq_stride = 0, cache_rows = 0, row_offset = 0;
    const int32_t *positions = nullptr;
    const float *rope_cos = nullptr, *rope_sin = nullptr;   // optional [n_seq * n_rows][32]
};
struct QueryJobArgs {
    const uint16_t *q = nullptr;
    const float *w = nullptr;
    int64_t n_rows = 0;
    uint8_t *q_fp8 = nullptr;
    float *w_eff = nullptr, *q_scale = nullptr;
    int32_t heads = 0;                                      // rows per token (for the RoPE tables)
    const float *rope_cos = nullptr, *rope_sin = nullptr;   // optional [n_rows / heads][32]
};

// Events armed by lk_profile_next_launch for the calling thread's next launch.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents &armed_events();

// Debug builds (-DLK_POISON_LDS) fill a kernel's shared objects with 0xFF bytes -- NaN as
// float32, f16 and e4m3fn -- before their first use, so that a read of LDS no thread has
// written turns into a parity failure.  Every thread of the block takes part and the
// fill ends with a barrier, so the call comes first in the kernel, ahead of any return.
#ifdef LK_POISON_LDS
__device__ __forceinline__ void poison_lds_bytes(void *p, size_t n) {
    if ((reinterpret_cast<uintptr_t>(p) & 3) == 0) {
        uint32_t *w = static_cast<uint32_t *>(p);
        for (size_t i = threadIdx.x; i < n / 4; i += blockDim.x) w[i] = 0xFFFFFFFFu;
        for (size_t i = n / 4 * 4 + threadIdx.x; i < n; i += blockDim.x) static_cast<uint8_t *>(p)[i] = 0xFF;
    } else {
        for (size_t i = threadIdx.x; i < n; i += blockDim.x) static_cast<uint8_t *>(p)[i] = 0xFF;
    }
}
template <typename... Objs>
__device__ __forceinline__ void poison_lds(Objs &...objs) {
    (poison_lds_bytes(static_cast<void *>(&objs), sizeof(objs)), ...);
    __syncthreads();
}
#define LK_POISON_LDS_OBJS(...) ::lk::poison_lds(__VA_ARGS__)
#else
#define LK_POISON_LDS_OBJS(...) ((void)0)
#endif

// Launch on `stream`; if events are armed, they are recorded at the kernel's own start
// and end (hipExtLaunchKernel) and disarmed.  Returns the status of this launch call
// itself (not an error left pending by earlier, unrelated HIP calls).  The arguments
// are converted to the kernel's parameter types before their addresses are taken.
template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t shm, hipStream_t stream,
                  Args... args) {
    static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
    std::tuple<Params...> vals{static_cast<Params>(args)...};
    void *argv[sizeof...(Params) > 0 ? sizeof...(Params) : 1] = {};
    std::apply([&argv](auto &...v) {
        int i = 0;
        ((argv[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    LaunchEvents &ev = armed_events();
    if (ev.start && ev.stop) {
        const LaunchEvents use = ev;
        ev = LaunchEvents{};
        return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, shm, stream,
                                  use.start, use.stop, 0);
    }
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, shm, stream);
}

}  // namespace lk

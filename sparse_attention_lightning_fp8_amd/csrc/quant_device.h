// quant_device.h -- one 128-feature row through the indexer's rotation and fp8
// quantization (gfx950), shared by the key/query kernel and the fused decode kernel.
//
// rotate_activation + act_quant of Indexer.forward (page "Hadamard rotation":
// kbar = ktilde (1/sqrt 128) H_128, bf16 in and out; page "Index key cache": e4m3fn
// values with one float32 power-of-two scale per 128 features).
//
// Layout: 8 consecutive lanes own one row, 16 features per lane (feature
// i = 16 * (lane % 8) + e).  The Walsh-Hadamard butterflies run in fp64: the inputs
// have 8-bit significands, so every partial sum is exact whenever the row's
// magnitudes span at most 2^38, and the result does not depend on butterfly order.
// Bits 0-3 of the feature index are combined in registers, bits 4-6 across the 8
// lanes with xor-shuffles.  Every function here starts with fp contract(off): the
// rounding steps must happen exactly where they are written, whatever the including
// file's contraction setting.
#pragma once

#include "lk_device.h"

namespace lk {

constexpr double kRotScale = 0x1.6a09e667f3bcdp-4;  // fl64(128 ** -0.5)
constexpr float kSoftmaxScale = 0x1.6a09e6p-4f;     // fl32(128 ** -0.5)

__device__ __forceinline__ double bf16_bits_to_double(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

// Round to the nearest bf16 value, ties to even, straight from fp64.
__device__ __forceinline__ double round_to_bf16(double p) {
#pragma clang fp contract(off)
    int e = __builtin_amdgcn_frexp_exp(p) - 1;  // 2^e <= |p| < 2^(e+1); p == 0 gives -1
    e = e < -126 ? -126 : e;                    // bf16 subnormal spacing is 2^-133
    return __builtin_ldexp(__builtin_rint(__builtin_ldexp(p, 7 - e)), e - 7);
}

// e4m3fn code of q, |q| <= 448: nearest-even, sign kept, never NaN.
__device__ __forceinline__ uint32_t encode_e4m3(float q) {
#pragma clang fp contract(off)
    float a = __builtin_fabsf(q);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);  // subnormals: multiples of 2^-9 (8 -> 0x08 = 2^-6)
    } else {
        int e = __builtin_amdgcn_frexp_expf(a) - 1;    // 2^e <= a < 2^(e+1), -6 <= e <= 8
        uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
        code = (uint32_t)((e + 7) << 3) + m - 8;       // m == 16 carries into the exponent
    }
    return code | (__float_as_uint(q) >> 24 & 0x80u);
}

// Quantize the row owned by this 8-lane group.  `in` holds the lane's 16 bf16 bit
// patterns (8 dwords).  Returns the 16 codes packed in 4 dwords and the exponent j.
__device__ __forceinline__ void quantize_row16(const uint32_t in[8], uint32_t out[4], int &j_out) {
#pragma clang fp contract(off)
    double x[16];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        x[2 * i] = bf16_bits_to_double(in[i] & 0xFFFFu);
        x[2 * i + 1] = bf16_bits_to_double(in[i] >> 16);
    }
    // In-lane butterflies: feature-index bits 0..3.
#pragma unroll
    for (int b = 1; b < 16; b <<= 1) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            if (e & b) continue;
            double u = x[e], v = x[e | b];
            x[e] = u + v;
            x[e | b] = u - v;
        }
    }
    // Cross-lane butterflies: feature-index bits 4..6 = lane bits 0..2.
    const int lane = __lane_id();
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 16; e++) {
            double y = __shfl_xor(x[e], m, 64);
            x[e] = upper ? (y - x[e]) : (x[e] + y);
        }
    }
    // Scale, round to bf16, amax.
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
        double r = x[e] == 0.0 ? 0.0 : x[e];   // an exact zero sum is +0
        double y = round_to_bf16(r * kRotScale);
        x[e] = y;
        amax = __builtin_fmax(amax, __builtin_fabs(y));
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) amax = __builtin_fmax(amax, __shfl_xor(amax, m, 64));
    // Smallest j >= -126 with amax <= 448 * 2^j.  amax = f * 2^E with f in [0.5, 1):
    // j = E - 9 if f <= 0.875 (448 = 0.875 * 2^9), else E - 8.
    int j = -126;
    if (amax > 0.0) {
        int E = __builtin_amdgcn_frexp_exp(amax);
        double f = __builtin_amdgcn_frexp_mant(amax);
        j = E - 9 + (f > 0.875 ? 1 : 0);
        j = j < -126 ? -126 : j;
    }
    j_out = j;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            float q = (float)__builtin_ldexp(x[4 * i + k], -j);  // exact for every value that can encode nonzero
            w |= encode_e4m3(q) << (8 * k);
        }
        out[i] = w;
    }
}

// Folded query weight of page "Index scores": fl32(fl32(w * 2^j) * fl32(128^-0.5)).
__device__ __forceinline__ float fold_weight(float w, int j) {
    const float ws = __fmul_rn(w, __builtin_ldexpf(1.0f, j));   // exact unless it leaves the float range
    return __fmul_rn(ws, kSoftmaxScale);
}

}  // namespace lk

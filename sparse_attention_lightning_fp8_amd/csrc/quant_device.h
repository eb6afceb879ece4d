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
// lanes with xor-shuffles (ds_bpermute or DPP, see cross_stage).  Every function here starts with fp contract(off): the
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

// e4m3fn codes of two floats with |q| <= 448 packed into half kHi of `old`:
// v_cvt_scalef32_pk_fp8_f32 with scale 1 rounds to nearest even and keeps the sign of
// values that round to zero; it agrees with the OCP e4m3fn encoding on every finite
// bf16 value in [-448, 448], subnormals included (checked exhaustively on gfx950).
// Every value quantized here has bf16 precision and magnitude at most 448.
typedef short lk_v2i16 __attribute__((ext_vector_type(2)));
template <bool kHi>
__device__ __forceinline__ lk_v2i16 encode_e4m3_pair(lk_v2i16 old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, 1.0f, kHi);
}

// A rotated feature (its exact Hadamard sum) times 128^-0.5 in one rounding, with an
// exact zero sum (of either sign) made +0: r * C + (+0) rounds the product once and
// turns only a -0 into +0, since a nonzero product plus zero is itself.  The fma is not
// folded into a plain multiply (that would keep -0).
__device__ __forceinline__ double scale_rot(double r) {
    return __builtin_fma(r, kRotScale, 0.0);
}

// scale_rot, then one rounding to bf16.
__device__ __forceinline__ double scale_round(double r) {
#pragma clang fp contract(off)
    return round_to_bf16(scale_rot(r));
}

// Nearest even to 8 significant bits straight on the fp64 bits (add half an ulp at
// bit 45, less one, plus the kept lowest bit, then clear bits 0-44): round_to_bf16 for
// every p that is zero or at least 2^-126 in magnitude (a normal bf16 magnitude), a
// carry into the exponent included.  Below 2^-126 it keeps more bits than bf16 has
// there, and its magnitude stays at most 2^-126.
__device__ __forceinline__ double round_to_bf16_normal(double p) {
    uint64_t u = (uint64_t)__double_as_longlong(p);
    u += 0xFFFFFFFFFFFull + ((u >> 45) & 1u);
    u &= ~0x1FFFFFFFFFFFull;
    return __longlong_as_double((long long)u);
}

// One cross-lane butterfly output: y - x in the upper lane of a pair, x + y in the
// lower, as fma(x, -1 or +1, y).  Multiplying by -1 is exact and the fma rounds once,
// so the result has the bits of the subtraction or the addition (signed zeros
// included), in one instruction.
__device__ __forceinline__ double butterfly_out(double x, double sign, double y) {
    return __builtin_fma(x, sign, y);
}

// Smallest j >= -126 with amax <= 448 * 2^j.  amax = f * 2^E with f in [0.5, 1):
// j = E - 9 if f <= 0.875 (448 = 0.875 * 2^9), else E - 8.
__device__ __forceinline__ int scale_exponent(double amax) {
    int j = -126;
    if (amax > 0.0) {
        const int E = __builtin_amdgcn_frexp_exp(amax);
        const double f = __builtin_amdgcn_frexp_mant(amax);
        j = E - 9 + (f > 0.875 ? 1 : 0);
        j = j < -126 ? -126 : j;
    }
    return j;
}

// Value of lane (lane ^ kM), kM = 1 .. 32: DPP quad_perm for 1 and 2, row_shl:4 /
// row_shr:4 for 4, row_ror:8 for 8 (within a 16-lane row, lane i + 8 mod 16 is i ^ 8),
// v_permlane16_swap for 16 (it returns rows (0, 0, 2, 2) and (1, 1, 3, 3)), and
// v_permlane32_swap for 32 (the low half twice, the high half twice).
template <int kM>
__device__ __forceinline__ uint32_t wave_xor_u32(uint32_t x) {
    const int lane = __lane_id();
    if constexpr (kM == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    } else if constexpr (kM == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
    } else if constexpr (kM == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x104, 0xF, 0xF, false);
        const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
        return (lane & 4) ? dn : up;
    } else if constexpr (kM == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
    } else if constexpr (kM == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? p[0] : p[1];
    } else {
        static_assert(kM == 32, "xor distance 1 .. 32");
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? p[0] : p[1];
    }
}
template <int kM>
__device__ __forceinline__ double wave_xor_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint64_t lo = wave_xor_u32<kM>((uint32_t)u), hi = wave_xor_u32<kM>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}
// One cross-lane butterfly stage of quantize_row16 (lane xor kM, kM = 1, 2 or 4) and
// the matching step of the row's max.  The first kDppStages stages read the partner
// through DPP quad_perm (VALU), the others through ds_bpermute (LDS): the preparation
// kernel is bound by its LDS issue and moves two stages to DPP; the fused decode
// kernel, whose VALU is the tighter pipe there, keeps all three on LDS.
template <int kM, int kDppStages>
__device__ __forceinline__ double lane_xor_f64(double x) {
    if constexpr (kM < (1 << kDppStages)) return wave_xor_f64<kM>(x);
    else return __shfl_xor(x, kM, 64);
}
template <int kM, int kDppStages>
__device__ __forceinline__ void cross_stage(double (&x)[16]) {
    const double sign = (__lane_id() & kM) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < 16; e++) x[e] = butterfly_out(x[e], sign, lane_xor_f64<kM, kDppStages>(x[e]));   // upper: y - x; lower: x + y
}

// Quantize the row owned by this 8-lane group.  `in` holds the lane's 16 bf16 bit
// patterns (8 dwords).  Returns the 16 codes packed in 4 dwords and the exponent j.
// kDppStages: see cross_stage (the results do not depend on it).
template <int kDppStages = 0>
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
    cross_stage<1, kDppStages>(x);
    cross_stage<2, kDppStages>(x);
    cross_stage<4, kDppStages>(x);
    // Scale and round to bf16 (scale_round), and the row's amax.  An exact zero sum can
    // come out of the butterflies as -0 in any row (a sum or difference of zeros drawn
    // from -0 inputs, such as a zero RoPE pair with a negative cosine, next to nonzero
    // features elsewhere), so scale_rot makes every exact zero +0 here, as the
    // definition's sum is.  (A nonzero p that rounds to zero keeps its sign.)
    // The bit rounding is exact for every nonzero |p| >= 2^-126.  A nonzero p below
    // that only matters when the scale exponent is -117 or less (otherwise both
    // roundings, at most 2^-126 in magnitude, times 2^-j <= 2^-10, encode to a zero of
    // p's sign), which needs amax <= 448 * 2^-117 < 2^-108; rows with a smaller amax
    // (zero rows included) take the exact rounding.  Rounding is monotone and odd, so
    // the row's amax is the rounding of max |p|.
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
        x[e] = scale_rot(x[e]);
        amax = __builtin_fmax(amax, __builtin_fabs(x[e]));
    }
    amax = __builtin_fmax(amax, lane_xor_f64<1, kDppStages>(amax));
    amax = __builtin_fmax(amax, lane_xor_f64<2, kDppStages>(amax));
    amax = __builtin_fmax(amax, lane_xor_f64<4, kDppStages>(amax));
    if (__any(amax < 0x1p-108)) {
#pragma unroll
        for (int e = 0; e < 16; e++) x[e] = round_to_bf16(x[e]);
        amax = round_to_bf16(amax);
    } else {
#pragma unroll
        for (int e = 0; e < 16; e++) x[e] = round_to_bf16_normal(x[e]);
        amax = round_to_bf16_normal(amax);
    }
    const int j = scale_exponent(amax);
    j_out = j;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float q[4];
#pragma unroll
        for (int k = 0; k < 4; k++) q[k] = (float)__builtin_ldexp(x[4 * i + k], -j);  // exact for every value that can encode nonzero
        lk_v2i16 w = {0, 0};
        w = encode_e4m3_pair<false>(w, q[0], q[1]);
        w = encode_e4m3_pair<true>(w, q[2], q[3]);
        out[i] = __builtin_bit_cast(uint32_t, w);
    }
}

// RoPE of Indexer.forward on the leading 64 features of the row owned by this 8-lane
// group ("rope in indexer is not interleaved": feature i pairs with i + 32).  `in`
// holds the lane's 16 bf16 features 16 * sub .. 16 * sub + 15 (two per dword); the
// partner features of lanes 0 and 1 live in lanes 2 and 3.  Products and sums are
// rounded in fp32 (no fused multiply-add), then each result once to bf16.  Lanes 4-7
// keep their features.

// This lane's 16 cosines and sines (pairs 16 * (sub % 2) + e) of one token's table
// row.  Every lane loads (lanes 4-7 read the same rows and ignore them), so callers
// can issue these loads ahead of others without a branch.
struct Rope16 {
    float c[16], s[16];
};
__device__ __forceinline__ void load_rope16(const float *__restrict__ cos_row, const float *__restrict__ sin_row,
                                            int sub, Rope16 &r) {
    const float4 *c4 = reinterpret_cast<const float4 *>(cos_row + 16 * (sub & 1));
    const float4 *s4 = reinterpret_cast<const float4 *>(sin_row + 16 * (sub & 1));
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const float4 cv = c4[q], sv = s4[q];
        r.c[4 * q] = cv.x; r.c[4 * q + 1] = cv.y; r.c[4 * q + 2] = cv.z; r.c[4 * q + 3] = cv.w;
        r.s[4 * q] = sv.x; r.s[4 * q + 1] = sv.y; r.s[4 * q + 2] = sv.z; r.s[4 * q + 3] = sv.w;
    }
}

// A whole table row (32 cosines, 32 sines) read through a block-uniform address, so
// the loads go through the scalar path and each lane picks its 16 with pick_rope16.
struct Rope32 {
    float c[32], s[32];
};
typedef const float __attribute__((address_space(4))) *const_f32_ptr;
__device__ __forceinline__ void load_rope32_uniform(const float *__restrict__ cos_row,
                                                    const float *__restrict__ sin_row, Rope32 &r) {
    // The tables are read-only for the kernel's lifetime, so the constant address
    // space is valid for them; with a uniform address that makes them scalar loads.
    const const_f32_ptr c = (const_f32_ptr)(uintptr_t)cos_row;
    const const_f32_ptr sn = (const_f32_ptr)(uintptr_t)sin_row;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        r.c[i] = c[i];
        r.s[i] = sn[i];
    }
}
__device__ __forceinline__ void pick_rope16(const Rope32 &all, int sub, Rope16 &r) {
    const bool hi = (sub & 1) != 0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
        r.c[e] = hi ? all.c[16 + e] : all.c[e];
        r.s[e] = hi ? all.s[16 + e] : all.s[e];
    }
}

// Every lane of the group must call it (it exchanges registers with lane sub ^ 2).
// Lanes 0-1 hold x_i and compute x_i c - x_{i+32} s, lanes 2-3 hold x_{i+32} and
// compute x_i s + x_{i+32} c; both are own * c + (+-(other * s)), bit for bit (the
// difference is the sum with the negated product, and addition commutes).  The bf16
// rounding is v_cvt_pk_bf16_f32, which equals round-to-nearest-even on the float's
// bits for every non-NaN input (checked exhaustively on gfx950).
typedef __bf16 lk_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void rope_row16(uint32_t in[8], const Rope16 &r, int sub) {
#pragma clang fp contract(off)
    uint32_t partner[8];
#pragma unroll
    for (int i = 0; i < 8; i++) partner[i] = (uint32_t)__shfl_xor((int)in[i], 2, 64);
    if (sub >= 4) return;
    const uint32_t flip = sub < 2 ? 0x80000000u : 0u;  // negate the other feature's product in lanes 0-1
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float y[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int e = 2 * i + h;
            const float own = __uint_as_float(((in[i] >> (16 * h)) & 0xFFFFu) << 16);
            const float oth = __uint_as_float(((partner[i] >> (16 * h)) & 0xFFFFu) << 16);
            const float os = __uint_as_float(__float_as_uint(oth * r.s[e]) ^ flip);
            y[h] = own * r.c[e] + os;
        }
        const lk_bf16x2 b = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){y[0], y[1]}, lk_bf16x2);
        in[i] = __builtin_bit_cast(uint32_t, b);
    }
}

// ---- One row spread over a whole wave (the fused decode kernel's new key): lane l
// holds features 2l and 2l + 1, feature-index bit 0 in registers and bits 1-6 as lane
// bits 0-5.  Lanes exchange through VALU only (DPP and permlane swaps), so the row
// costs one wave a few hundred cycles instead of a full 16-feature pass.  Every lane
// of the wave must take part (full EXEC).

template <int kM>
__device__ __forceinline__ void wave_butterfly(double &x0, double &x1) {
#pragma clang fp contract(off)
    const double sign = (__lane_id() & kM) ? -1.0 : 1.0;
    const double y0 = wave_xor_f64<kM>(x0), y1 = wave_xor_f64<kM>(x1);
    x0 = butterfly_out(x0, sign, y0);                      // upper: y - x; lower: x + y
    x1 = butterfly_out(x1, sign, y1);
}

// Returns this lane's two codes in bits 0-15 (feature 2l in the low byte) and the
// row's exponent j (the same in every lane).  Arithmetic as quantize_row16.
__device__ __forceinline__ uint32_t quantize_row_wave(uint32_t in, int &j_out) {
#pragma clang fp contract(off)
    double x0 = bf16_bits_to_double(in & 0xFFFFu), x1 = bf16_bits_to_double(in >> 16);
    const double u = x0 + x1, v = x0 - x1;            // feature-index bit 0
    x0 = u;
    x1 = v;
    wave_butterfly<1>(x0, x1);
    wave_butterfly<2>(x0, x1);
    wave_butterfly<4>(x0, x1);
    wave_butterfly<8>(x0, x1);
    wave_butterfly<16>(x0, x1);
    wave_butterfly<32>(x0, x1);
    x0 = scale_round(x0);
    x1 = scale_round(x1);
    double amax = __builtin_fmax(__builtin_fabs(x0), __builtin_fabs(x1));
    amax = __builtin_fmax(amax, wave_xor_f64<1>(amax));
    amax = __builtin_fmax(amax, wave_xor_f64<2>(amax));
    amax = __builtin_fmax(amax, wave_xor_f64<4>(amax));
    amax = __builtin_fmax(amax, wave_xor_f64<8>(amax));
    amax = __builtin_fmax(amax, wave_xor_f64<16>(amax));
    amax = __builtin_fmax(amax, wave_xor_f64<32>(amax));
    const int j = scale_exponent(amax);
    j_out = j;
    lk_v2i16 w = {0, 0};
    w = encode_e4m3_pair<false>(w, (float)__builtin_ldexp(x0, -j), (float)__builtin_ldexp(x1, -j));
    return (uint32_t)(uint16_t)w[0];
}

// RoPE in the wave layout: feature i < 32 (lanes 0-15) pairs with i + 32 (lanes
// 16-31, lane xor 16); c and s are this lane's two table entries, pairs
// 2 (lane % 16) and 2 (lane % 16) + 1.  Same rounding as rope_row16.
__device__ __forceinline__ void rope_row_wave(uint32_t &in, float2 c, float2 s) {
#pragma clang fp contract(off)
    const uint32_t partner = wave_xor_u32<16>(in);
    const int lane = __lane_id();
    if (lane >= 32) return;
    const uint32_t flip = lane < 16 ? 0x80000000u : 0u;
    const float cc[2] = {c.x, c.y}, ss[2] = {s.x, s.y};
    float y[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const float own = __uint_as_float(((in >> (16 * h)) & 0xFFFFu) << 16);
        const float oth = __uint_as_float(((partner >> (16 * h)) & 0xFFFFu) << 16);
        y[h] = own * cc[h] + __uint_as_float(__float_as_uint(oth * ss[h]) ^ flip);
    }
    const lk_bf16x2 b = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){y[0], y[1]}, lk_bf16x2);
    in = __builtin_bit_cast(uint32_t, b);
}

// Folded query weight of page "Index scores": fl32(fl32(w * 2^j) * fl32(128^-0.5)).
__device__ __forceinline__ float fold_weight(float w, int j) {
    const float ws = __fmul_rn(w, __builtin_ldexpf(1.0f, j));   // exact unless it leaves the float range
    return __fmul_rn(ws, kSoftmaxScale);
}

}  // namespace lk

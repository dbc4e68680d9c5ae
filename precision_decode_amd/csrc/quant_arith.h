// Scalar arithmetic of the BF16 -> NVFP4 quantiser on gfx950: bf16 unpacking,
// the E4M3 block-scale encode and decode, and the correctly rounded quotients
// it takes without a division, each exact where the quantiser uses it (the
// CuTeDSL NVFP4 bridge page, section "Quantization", fixes the IEEE fp32
// operations they stand for).  Device code only, shared by the quantiser
// kernel (nvfp4_quantize.hip) and the device checks that compare these forms
// with IEEE division over the whole range where the quantiser relies on them.
#ifndef NVFP4_QUANT_ARITH_H
#define NVFP4_QUANT_ARITH_H

#include <hip/hip_runtime.h>

#include <cstdint>

namespace nvfp4quant {

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> E4M3 (float8_e4m3fn) code for v > 0, or NaN / +Inf: round to
// nearest even; values from 464 up (halfway to the first step past 448, whose
// pattern is NaN), infinities and NaN give 0x7F.
__device__ __forceinline__ uint32_t e4m3_code_pos(float v) {
    if (!(v <= 464.0f)) return 0x7Fu;
    if (v < 0.015625f) {                         // below 2^-6: subnormal steps of 2^-9
        return static_cast<uint32_t>(__builtin_rintf(v * 512.0f));   // exact scaling, 0..8
    }
    // normal: keep 3 mantissa bits with round-to-nearest-even on the fp32 pattern
    const uint32_t b = __float_as_uint(v);
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;     // (exp << 3 | mant), rounded
    return r - (120u << 3);                       // rebias 127 -> 7
}

// E4M3 code (0..0x7F, sign clear) -> float; 0x7F is NaN.
__device__ __forceinline__ float e4m3_value_pos(uint32_t s) {
    if (s == 0x7Fu) return __uint_as_float(0x7FC00000u);
    if (s < 8u) return static_cast<float>(s) * 0.001953125f;          // s * 2^-9, exact
    return __uint_as_float((((s >> 3) + 120u) << 23) | ((s & 7u) << 20));
}

// RN32(a / b) from y within one fp64 ulp of 1/b as RN32(RN64(a * y)): the
// fp64 product is within 2^-51 (relative) of a/b, so this is exact whenever
// a/b, if not representable, lies farther than that from every fp32 rounding
// midpoint and is not a subnormal fp32 number.
__device__ __forceinline__ float quot_f64(float a, double y) {
    return static_cast<float>(static_cast<double>(a) * y);
}

// 1/d within one fp64 ulp for a normal d far from the exponent range's ends:
// two Newton steps from the hardware reciprocal (relative error below 2^-22),
// each step squaring the error; the fused residual 1 - d y is exact to well
// under an ulp of itself, so the last step's rounding is the only one left.
__device__ __forceinline__ double recip_f64(double d) {
    double y = __builtin_amdgcn_rcp(d);
    double e = __builtin_fma(-d, y, 1.0);
    y = __builtin_fma(y, e, y);
    e = __builtin_fma(-d, y, 1.0);
    return __builtin_fma(y, e, y);
}

// RN32(a / b) for b with at most 4 significant bits, from y within 2^-22 of
// 1/b: q = RN(a*y) is within 2^-21 of a/b, the residual a - b*q is exact, and
// one correction lands within 2^-42 of a/b, far closer than the 2^-29 that
// separates a/b from any rounding midpoint; a zero quotient comes out as +0.
__device__ __forceinline__ float quot_short(float a, float b, float y) {
    const float q = a * y;
    const float e = __builtin_fmaf(-b, q, a);
    return __builtin_fmaf(e, y, q);
}

// Half-step rounding (see block_codes in nvfp4_quantize.hip): f(a) = RN(a (1 - 2^-24)
// - 0.25 + 5 2^-24) as one fma.
constexpr float kHalfStepScale = 0x1.fffffep-1f;            // 1 - 2^-24
constexpr float kHalfStepShift = -0.25f + 5.0f * 0x1p-24f;  // exact in fp32

}  // namespace nvfp4quant

#endif  // NVFP4_QUANT_ARITH_H

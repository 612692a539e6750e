// exp2_poly.h -- 2^x in software on the FMA pipe, for gfx950 device code.
//
// The FlashAttention-4 section of "FlashAttention 1-4 evolution cheat sheet"
// (argus-lessons) computes part of the softmax exponentials with a polynomial
// on the FMA units instead of the hardware exponential unit.  This is that
// exponential, written from two published methods:
//   * Cody-Waite argument reduction (W. J. Cody and W. Waite, "Software
//     Manual for the Elementary Functions", 1980): x = j + f with j =
//     round(x) and |f| <= 1/2, so 2^x = 2^j * 2^f.  j is found by adding
//     1.5 * 2^23: the sum rounds x to an integer held in the low mantissa
//     bits, and subtracting the constant again gives j exactly, so f = x - j
//     is exact too.
//   * a minimax polynomial for 2^f on [-1/2, 1/2] (relative error,
//     equioscillating; Remez exchange algorithm), degree 3.  The
//     coefficients come from gen_exp2_poly.py beside this file; its maximum
//     relative error is 7.5e-5 in exact arithmetic.
// 2^j is applied by adding j << 23 to the bit pattern of the polynomial's
// value (an exponent add: v_lshl_add_u32), which is exact while the result
// stays a normal number.
//
// Domain: for -125 <= x <= 127 the result is a normal number within
// kExp2PolyRelErr of 2^x (the polynomial's error plus the fp32 rounding of
// three FMAs).  Below, x is clamped at -126 so that the exponent add never
// wraps (the polynomial's value at f = 0 is just under 1, so j = -127 would
// carry into the sign and exponent bits and make a NaN): every x < -125,
// -inf included, gives a non-negative value below 2^-124, possibly a
// subnormal bit pattern that is not close to 2^x.  At that size a
// probability is nothing next to a row whose largest term is at least 1;
// masked keys are set to 0 separately.  Cost: 8 VALU instructions (max, add, sub, sub,
// three FMAs, lshl_add) against one v_exp_f32.
#pragma once

#include <stdint.h>

namespace attn_gfx950 {

constexpr float kExp2C0 = 0.9999280571937561f;
constexpr float kExp2C1 = 0.69326096773147583f;
constexpr float kExp2C2 = 0.2426111251115799f;
constexpr float kExp2C3 = 0.055171668529510498f;
// Stated bound of exp2_poly's relative error for x >= -125:
// the minimax error 7.5e-5 plus the fp32 rounding of the three FMAs.
constexpr float kExp2PolyRelErr = 1e-4f;

__device__ __forceinline__ float exp2_poly(float x)
{
    x = __builtin_fmaxf(x, -126.f);
    const float t = x + 12582912.f;  // 1.5 * 2^23: round(x) in the low mantissa bits
    const float j = t - 12582912.f;
    const float f = x - j;  // exact, |f| <= 1/2
    const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, kExp2C0);
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p) + (__builtin_bit_cast(uint32_t, t) << 23));
}

}  // namespace attn_gfx950

// mx.hpp - OCP microscaling FP4 (MXFP4) element and block-scale rules shared by
// the kernels that quantize rotated rows (the W4A4 extension's MXFP4 variant;
// "ParoQuant" blog, Bits and formats).
//
// A block of 32 consecutive values shares an E8M0 scale byte b (2^(b - 127)),
// b = floor(log2 max|v|) - 2 + 127, 0 for a zero or tiny block; values are
// E2M1 codes (bit 3 sign; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) of
// v / 2^(b - 127), nearest with ties to the even code, clamped at 6, zero as +0.
#pragma once

#include "common.hpp"

namespace paro {

// E2M1 code of a (already divided by the block scale): the count of rounding
// boundaries below |a|, ties to the even code (0, 1.0, 1.0, 2.0, 2.0, 4.0,
// 4.0), saturating at 6; sign in bit 3 unless the magnitude is zero.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  const float m = fabsf(a);
  const uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) + (uint32_t)(m >= 1.75f) +
                     (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
  return (a < 0.0f && c != 0) ? (c | 8u) : c;
}

// Biased E8M0 exponent of a block whose largest magnitude is amax (fp32):
// floor(log2 amax) is the exponent field minus 127 for a normal amax.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return amax > 0.0f && ef > 2 ? ef - 2 : 0;
}

// v divided by the block scale 2^(biased - 127), exactly
__device__ __forceinline__ float mx_scaled(float v, int biased) { return __builtin_ldexpf(v, 127 - biased); }

}  // namespace paro

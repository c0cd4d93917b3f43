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

// E2M1 codes of two values already divided by the block scale, as one byte
// (a in the low nibble).  The CDNA4 format conversion (divisor 1.0) rounds to
// the nearest code with ties to the even one and saturates at 6, which is the
// rule above; a negative value that rounds to zero keeps its sign bit there,
// so that bit is cleared (zero is stored as +0).
__device__ __forceinline__ uint32_t e2m1_pair(float a, float b) {
  const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xffu;
  const uint32_t nz = ((r & 0x77u) + 0x77u) & 0x88u;  // bit 3 of each nibble whose magnitude is nonzero
  return r & (nz | 0x77u);
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

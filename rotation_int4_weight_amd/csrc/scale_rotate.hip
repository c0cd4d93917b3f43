// scale_rotate.hip - channel scaling + pairwise Givens rotation of activations.
//
// "ParoQuant" wiki, Concepts / Activation and weight transforms: X_r = X D^-1 R
// with the stored channel_scales equal to D^-1 (multiplied in); Concepts /
// Pairwise Givens rotations: krot ordered stages of disjoint pair rotations,
// local to each 128-channel group.
//
// One workgroup = 4 waves on one group g and up to 4*TW token rows; each wave
// stages TW rows x 128 channels of the group in LDS (fp32), applies every
// stage with the pair/angle of lane p held in registers, and writes the rows
// back out coalesced (lane p owns channels 2p and 2p+1 on load and store).
#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kRotTW = 16;       // token rows per wave
constexpr int kRotRS = kG + 4;   // LDS row stride (floats), staggers banks across rows

template <int XDT, int ODT>
__global__ void __launch_bounds__(256)
scale_rotate_kernel(const uint16_t *__restrict__ x, void *__restrict__ xr, int64_t tokens, int64_t I,
                    const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                    const float *__restrict__ cscale, int krot) {
  __shared__ float lds[4][kRotTW * kRotRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t m0 = ((int64_t)blockIdx.y * 4 + wave) * kRotTW;
  if (m0 >= tokens) return;  // whole wave idle (no block-level barrier below)
  const int T = (int)((tokens - m0) < kRotTW ? (tokens - m0) : kRotTW);
  float *xs = lds[wave];
  const int64_t c0 = g * kG + 2 * lane;

  // load + channel scale (x . D^-1)
  const float s0 = cscale[c0], s1 = cscale[c0 + 1];
#pragma unroll
  for (int m = 0; m < kRotTW; ++m) {
    if (m < T) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(x + (m0 + m) * I + c0);
      xs[m * kRotRS + 2 * lane] = act_to_f32<XDT>(w & 0xffffu) * s0;
      xs[m * kRotRS + 2 * lane + 1] = act_to_f32<XDT>(w >> 16) * s1;
    }
  }
  wave_lds_sync();

  rotate_rows_lds<kRotTW>(xs, kRotRS, T, pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane);

#pragma unroll
  for (int m = 0; m < kRotTW; ++m) {
    if (m < T) {
      const float a = xs[m * kRotRS + 2 * lane], b = xs[m * kRotRS + 2 * lane + 1];
      const int64_t o = (m0 + m) * I + c0;
      if constexpr (ODT == kF32) {
        *reinterpret_cast<float2 *>(reinterpret_cast<float *>(xr) + o) = make_float2(a, b);
      } else {
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(xr) + o) = pack2<ODT>(a, b);
      }
    }
  }
}

template <int XDT, int ODT>
static hipError_t launch_rot(const uint16_t *x, void *xr, int64_t tokens, int64_t I, const int16_t *pairs,
                             const float *theta, const float *cs, int krot, hipStream_t st) {
  const int64_t per_block = 4 * kRotTW;
  dim3 grid((unsigned)(I / kG), (unsigned)((tokens + per_block - 1) / per_block));
  hipLaunchKernelGGL((scale_rotate_kernel<XDT, ODT>), grid, dim3(256), 0, st, x, xr, tokens, I, pairs,
                     theta, cs, krot);
  return hipGetLastError();
}

hipError_t launch_scale_rotate(const uint16_t *x, int x_dt, void *xr, int xr_dt, int64_t tokens, int64_t I,
                               const int16_t *pairs, const float *theta, const float *cs, int krot,
                               hipStream_t st) {
  if (x_dt == kF16) {
    if (xr_dt == kF16) return launch_rot<kF16, kF16>(x, xr, tokens, I, pairs, theta, cs, krot, st);
    if (xr_dt == kBF16) return launch_rot<kF16, kBF16>(x, xr, tokens, I, pairs, theta, cs, krot, st);
    return launch_rot<kF16, kF32>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  }
  if (xr_dt == kF16) return launch_rot<kBF16, kF16>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  if (xr_dt == kBF16) return launch_rot<kBF16, kBF16>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  return launch_rot<kBF16, kF32>(x, xr, tokens, I, pairs, theta, cs, krot, st);
}

}  // namespace paro

// scale_rotate.hip - channel scaling + pairwise Givens rotation of activations.
//
// "ParoQuant" wiki, Concepts / Activation and weight transforms: X_r = X D^-1 R
// with the stored channel_scales equal to D^-1 (multiplied in); Concepts /
// Pairwise Givens rotations: krot ordered stages of disjoint pair rotations,
// local to each 128-channel group.
//
// One workgroup = 4 waves on one group g and up to 4*RW token rows; each wave
// stages RW rows x 128 channels of the group in LDS (fp32), applies every
// stage with the pair/angle of lane p held in registers, and writes the rows
// back out coalesced (lane p owns channels 2p and 2p+1 on load and store).
// RW is 16 for many tokens (the pair/angle loads and sin/cos are amortised
// over more rows) and 1..4 for few tokens (more waves, shorter chains of
// dependent LDS stages).
#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kRotRS = kG + 4;   // LDS row stride (floats), staggers banks across rows

template <int XDT, int ODT, int RW>
__global__ void __launch_bounds__(256)
scale_rotate_kernel(const uint16_t *__restrict__ x, void *__restrict__ xr, int64_t tokens, int64_t I,
                    const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                    const float *__restrict__ cscale, int krot) {
  __shared__ float lds[4][RW * kRotRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t m0 = ((int64_t)blockIdx.y * 4 + wave) * RW;
  if (m0 >= tokens) return;  // whole wave idle (no block-level barrier below)
  const int T = (int)((tokens - m0) < RW ? (tokens - m0) : RW);
  float *xs = lds[wave];
  const int64_t c0 = g * kG + 2 * lane;

  RotParams rp;
  rp.load(pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane);
  // load + channel scale (x . D^-1); rows past the last token are zero
  const float s0 = cscale[c0], s1 = cscale[c0 + 1];
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const int mm = m < T ? m : 0;
    const uint32_t w = *reinterpret_cast<const uint32_t *>(x + (m0 + mm) * I + c0);
    xs[m * kRotRS + 2 * lane] = m < T ? act_to_f32<XDT>(w & 0xffffu) * s0 : 0.0f;
    xs[m * kRotRS + 2 * lane + 1] = m < T ? act_to_f32<XDT>(w >> 16) * s1 : 0.0f;
  }
  wave_lds_sync();

  rotate_rows_lds<RW>(xs, kRotRS, rp, pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane);

#pragma unroll
  for (int m = 0; m < RW; ++m) {
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

// Same transform, output in the fragment-major tiled layout (launch.hpp):
// each wave holds one complete 16-row tile of group g (rows past the last
// token are zero) and writes its four 32-column blocks as 1 KB contiguous
// stores, lane L taking row L&15 and columns 8(L>>4)..+7 of each block.
template <int XDT>
__global__ void __launch_bounds__(256)
scale_rotate_tiled_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ xt, int64_t tokens, int64_t I,
                          const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                          const float *__restrict__ cscale, int krot) {
  constexpr int RW = 16;
  __shared__ float lds[4][RW * kRotRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t m0 = ((int64_t)blockIdx.y * 4 + wave) * RW;
  if (m0 >= tokens) return;  // whole tile past the padded end (no block-level barrier below)
  const int T = (int)((tokens - m0) < RW ? (tokens - m0) : RW);
  float *xs = lds[wave];
  const int64_t c0 = g * kG + 2 * lane;

  RotParams rp;
  rp.load(pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane);
  const float s0 = cscale[c0], s1 = cscale[c0 + 1];
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const int mm = m < T ? m : 0;
    const uint32_t w = *reinterpret_cast<const uint32_t *>(x + (m0 + mm) * I + c0);
    xs[m * kRotRS + 2 * lane] = m < T ? act_to_f32<XDT>(w & 0xffffu) * s0 : 0.0f;
    xs[m * kRotRS + 2 * lane + 1] = m < T ? act_to_f32<XDT>(w >> 16) * s1 : 0.0f;
  }
  wave_lds_sync();

  rotate_rows_lds<RW>(xs, kRotRS, rp, pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane);

  const int r = lane & 15, kb = lane >> 4;
  uint16_t *blk = xt + ((m0 / 16) * (I / 32) + g * (kG / 32)) * 512 + lane * 8;
#pragma unroll
  for (int q = 0; q < kG / 32; ++q) {
    const float *src = xs + r * kRotRS + 32 * q + 8 * kb;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pack2<XDT>(src[2 * e], src[2 * e + 1]);
    *reinterpret_cast<u32x4 *>(blk + q * 512) = v;
  }
}

hipError_t launch_scale_rotate_tiled(const uint16_t *x, int x_dt, uint16_t *xt, int64_t tokens, int64_t I,
                                     const int16_t *pairs, const float *theta, const float *cs, int krot,
                                     hipStream_t st) {
  dim3 grid((unsigned)(I / kG), (unsigned)((tokens + 63) / 64));
  if (x_dt == kF16)
    hipLaunchKernelGGL((scale_rotate_tiled_kernel<kF16>), grid, dim3(256), 0, st, x, xt, tokens, I, pairs, theta,
                       cs, krot);
  else
    hipLaunchKernelGGL((scale_rotate_tiled_kernel<kBF16>), grid, dim3(256), 0, st, x, xt, tokens, I, pairs, theta,
                       cs, krot);
  return hipGetLastError();
}

// Row-major -> tiled copy: a wave per 16 x 32 block (grid-stride), lane L
// moving row L&15, columns 8(L>>4)..+7 (zeros for rows past the last token).
__global__ void __launch_bounds__(256)
retile_kernel(const uint16_t *__restrict__ xr, uint16_t *__restrict__ xt, int64_t tokens, int64_t I,
              int64_t blocks) {
  const int lane = lane_id();
  const int64_t ksteps = I / 32;
  for (int64_t b = (int64_t)blockIdx.x * 4 + wave_id(); b < blocks; b += (int64_t)gridDim.x * 4) {
    const int64_t mt = b / ksteps, ks = b % ksteps;
    const int64_t m = mt * 16 + (lane & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < tokens) v = *reinterpret_cast<const u32x4 *>(xr + m * I + ks * 32 + (lane >> 4) * 8);
    *reinterpret_cast<u32x4 *>(xt + b * 512 + lane * 8) = v;
  }
}

hipError_t launch_retile(const uint16_t *xr, uint16_t *xt, int64_t tokens, int64_t I, hipStream_t st) {
  const int64_t blocks = tiled_rows(tokens) / 16 * (I / 32);
  const int64_t wgs = (blocks + 3) / 4;
  hipLaunchKernelGGL(retile_kernel, dim3((unsigned)(wgs < (1 << 20) ? wgs : (1 << 20))), dim3(256), 0, st, xr, xt,
                     tokens, I, blocks);
  return hipGetLastError();
}

template <int XDT, int ODT, int RW>
static hipError_t launch_rot_rw(const uint16_t *x, void *xr, int64_t tokens, int64_t I, const int16_t *pairs,
                                const float *theta, const float *cs, int krot, hipStream_t st) {
  const int64_t per_block = 4 * RW;
  dim3 grid((unsigned)(I / kG), (unsigned)((tokens + per_block - 1) / per_block));
  hipLaunchKernelGGL((scale_rotate_kernel<XDT, ODT, RW>), grid, dim3(256), 0, st, x, xr, tokens, I, pairs,
                     theta, cs, krot);
  return hipGetLastError();
}

template <int XDT, int ODT>
static hipError_t launch_rot(const uint16_t *x, void *xr, int64_t tokens, int64_t I, const int16_t *pairs,
                             const float *theta, const float *cs, int krot, hipStream_t st) {
  if (tokens <= 4) return launch_rot_rw<XDT, ODT, 1>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  if (tokens <= 64) return launch_rot_rw<XDT, ODT, 4>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  return launch_rot_rw<XDT, ODT, 16>(x, xr, tokens, I, pairs, theta, cs, krot, st);
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

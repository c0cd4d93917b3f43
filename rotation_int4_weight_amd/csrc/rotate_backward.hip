// rotate_backward.hip - backward of the channel scaling and pairwise rotation
// (the calibration step of the method: the optimizer updates angles and
// channel scales through the rotation; "ParoQuant" wiki, Straight-through
// estimation, and the pair formula of Concepts / Pairwise Givens rotations).
//
// For x_r = (x * cs) . R and an incoming gradient g = dL/dx_r:
//   per stage, backwards, with the stage's outputs (a', b') and gradients
//   (ga', gb') of a pair with angle theta:
//     dL/dtheta += ga' b' - gb' a'
//     (ga, gb)   = (ga' c - gb' s, ga' s + gb' c)
//   then dL/dx = gs * cs and dL/dcs = sum over tokens of gs * x, with gs the
//   gradient of the scaled rows.
//
// The stage outputs are not stored: each wave recomputes the forward of its
// 16 rows in LDS (fp32) and then, walking the stages back, inverts each stage
// ((a, b) = (a' c - b' s, a' s + b' c)) to recover its inputs while it
// propagates the gradient.  dL/dtheta and dL/dcs are sums over tokens: every
// wave writes its 16-row partial sums to the workspace, and a second kernel
// adds the partials in a fixed order (the result does not depend on
// scheduling).
#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kBRS = kG + 4;  // LDS row stride (floats)

template <int DT>
__device__ __forceinline__ float2 load_pair(const void *p, int64_t idx) {
  if constexpr (DT == kF32) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(p) + idx);
  } else {
    const uint32_t b = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(p) + idx);
    return float2{act_to_f32<DT>(b & 0xffffu), act_to_f32<DT>(b >> 16)};
  }
}

template <int DT>
__device__ __forceinline__ void store_pair(void *p, int64_t idx, float a, float b) {
  if constexpr (DT == kF32)
    *reinterpret_cast<float2 *>(reinterpret_cast<float *>(p) + idx) = float2{a, b};
  else
    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(p) + idx) = pack2<DT>(a, b);
}

// partial: [tiles * 4 waves][E] fp32, E = krot * I/2 (dtheta) + I (dcs)
template <int XDT, int GDT, int ODT>
__global__ void __launch_bounds__(256)
rot_backward_kernel(const void *__restrict__ x, const void *__restrict__ gin, int64_t tokens, int64_t I,
                    const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                    const float *__restrict__ cscale, int krot, void *__restrict__ gx, float *__restrict__ partial) {
  constexpr int RW = 16;
  __shared__ float lds[4][2][RW * kBRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * 64 + wave * RW;
  const int64_t E = (int64_t)krot * (I / 2) + I;
  float *prow = partial + ((int64_t)blockIdx.y * 4 + wave) * E;
  float *xs = lds[wave][0], *gs = lds[wave][1];
  const int16_t *pairs_g = pairs + g * kG;
  const float *theta_g = theta + g * kPairs;

  RotParams rp;
  rp.load(pairs_g, I, theta_g, I / 2, krot, lane);
  const float2 csv = *reinterpret_cast<const float2 *>(cscale + g * kG + 2 * lane);

  // rows past the last token are zero: they add nothing to the sums
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    float2 v{0.f, 0.f}, w{0.f, 0.f};
    if (m0 + m < tokens) {
      v = load_pair<XDT>(x, (m0 + m) * I + g * kG + 2 * lane);
      w = load_pair<GDT>(gin, (m0 + m) * I + g * kG + 2 * lane);
    }
    xs[m * kBRS + 2 * lane] = v.x * csv.x;
    xs[m * kBRS + 2 * lane + 1] = v.y * csv.y;
    gs[m * kBRS + 2 * lane] = w.x;
    gs[m * kBRS + 2 * lane + 1] = w.y;
  }
  wave_lds_sync();
  rotate_rows_lds<RW>(xs, kBRS, rp, pairs_g, I, theta_g, I / 2, krot, lane);  // xs = x_r

  // stages backwards: lane p owns pair p of every stage
  for (int t = krot - 1; t >= 0; --t) {
    uint32_t pw;
    float th;
    if (t < kStageRegs) {
      pw = rp.pw[0];
      th = rp.th[0];
#pragma unroll
      for (int u = 1; u < kStageRegs; ++u)
        if (t == u) {
          pw = rp.pw[u];
          th = rp.th[u];
        }
    } else {
      pw = *reinterpret_cast<const uint32_t *>(pairs_g + (int64_t)t * I + 2 * lane);
      th = theta_g[(int64_t)t * (I / 2) + lane];
    }
    float c, s;
    __sincosf(th, &s, &c);
    const int a = (int)(pw & (kG - 1)), b = (int)((pw >> 16) & (kG - 1));
    float dth = 0.0f;
#pragma unroll
    for (int m = 0; m < RW; ++m) {
      const float ap = xs[m * kBRS + a], bp = xs[m * kBRS + b];
      const float gap = gs[m * kBRS + a], gbp = gs[m * kBRS + b];
      dth = __builtin_fmaf(gap, bp, __builtin_fmaf(-gbp, ap, dth));
      xs[m * kBRS + a] = __builtin_fmaf(ap, c, -(bp * s));
      xs[m * kBRS + b] = __builtin_fmaf(ap, s, bp * c);
      gs[m * kBRS + a] = __builtin_fmaf(gap, c, -(gbp * s));
      gs[m * kBRS + b] = __builtin_fmaf(gap, s, gbp * c);
    }
    prow[(int64_t)t * (I / 2) + g * kPairs + lane] = dth;
    wave_lds_sync();
  }

  // dL/dx = gs * cs; partial dL/dcs = sum over the rows of gs * x
  float dc0 = 0.0f, dc1 = 0.0f;
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    if (m0 + m >= tokens) break;
    const float g0 = gs[m * kBRS + 2 * lane], g1 = gs[m * kBRS + 2 * lane + 1];
    const float2 v = load_pair<XDT>(x, (m0 + m) * I + g * kG + 2 * lane);
    dc0 = __builtin_fmaf(g0, v.x, dc0);
    dc1 = __builtin_fmaf(g1, v.y, dc1);
    store_pair<ODT>(gx, (m0 + m) * I + g * kG + 2 * lane, g0 * csv.x, g1 * csv.y);
  }
  *reinterpret_cast<float2 *>(prow + (int64_t)krot * (I / 2) + g * kG + 2 * lane) = float2{dc0, dc1};
}

// out[e] = sum over p < P of partial[p][e], in order of p
__global__ void __launch_bounds__(256)
rot_backward_reduce_kernel(const float *__restrict__ partial, int64_t P, int64_t E, float *__restrict__ gtheta,
                           int64_t n_theta, float *__restrict__ gcs) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  float s = 0.0f;
  for (int64_t p = 0; p < P; ++p) s += partial[p * E + e];
  if (e < n_theta)
    gtheta[e] = s;
  else
    gcs[e - n_theta] = s;
}

size_t rot_backward_partial_bytes(int64_t tokens, int64_t I, int krot) {
  const int64_t tiles = (tokens + 63) / 64;
  return (size_t)(tiles * 4) * (size_t)((int64_t)krot * (I / 2) + I) * 4;
}

template <int XDT, int GDT>
static void launch_bwd_o(int gx_dt, dim3 grid, hipStream_t st, const void *x, const void *gin, int64_t tokens,
                         int64_t I, const int16_t *pairs, const float *theta, const float *cs, int krot, void *gx,
                         float *partial) {
  if (gx_dt == kF32)
    hipLaunchKernelGGL((rot_backward_kernel<XDT, GDT, kF32>), grid, dim3(256), 0, st, x, gin, tokens, I, pairs, theta,
                       cs, krot, gx, partial);
  else
    hipLaunchKernelGGL((rot_backward_kernel<XDT, GDT, XDT>), grid, dim3(256), 0, st, x, gin, tokens, I, pairs, theta,
                       cs, krot, gx, partial);
}

template <int XDT>
static void launch_bwd_g(int g_dt, int gx_dt, dim3 grid, hipStream_t st, const void *x, const void *gin,
                         int64_t tokens, int64_t I, const int16_t *pairs, const float *theta, const float *cs, int krot,
                         void *gx, float *partial) {
  if (g_dt == kF32)
    launch_bwd_o<XDT, kF32>(gx_dt, grid, st, x, gin, tokens, I, pairs, theta, cs, krot, gx, partial);
  else
    launch_bwd_o<XDT, XDT>(gx_dt, grid, st, x, gin, tokens, I, pairs, theta, cs, krot, gx, partial);
}

hipError_t launch_rot_backward(const void *x, int x_dt, const void *gin, int g_dt, int64_t tokens, int64_t I,
                               const int16_t *pairs, const float *theta, const float *cs, int krot, void *gx,
                               int gx_dt, float *gtheta, float *gcs, float *partial, hipStream_t st) {
  const int64_t tiles = (tokens + 63) / 64;
  if (tiles > 0) {  // with no tokens the sums below are zero
    const dim3 grid((unsigned)(I / kG), (unsigned)tiles);
    if (x_dt == kF16)
      launch_bwd_g<kF16>(g_dt, gx_dt, grid, st, x, gin, tokens, I, pairs, theta, cs, krot, gx, partial);
    else
      launch_bwd_g<kBF16>(g_dt, gx_dt, grid, st, x, gin, tokens, I, pairs, theta, cs, krot, gx, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t E = (int64_t)krot * (I / 2) + I;
  hipLaunchKernelGGL(rot_backward_reduce_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, st, partial,
                     tiles * 4, E, gtheta, (int64_t)krot * (I / 2), gcs);
  return hipGetLastError();
}

}  // namespace paro

// quantize.hip - the offline side of the method: transform a dense weight into
// the rotated domain, quantize it group-wise to four bits and pack it in the
// stored AWQ layout.
//
//   W_r = W . D . R          ("ParoQuant" wiki, Concepts / Activation and weight
//                             transforms; W is [O][I], the stored channel
//                             scales are D^-1, so they divide W's input
//                             channels; R is the staged rotation)
//   per output row n and group g of G input channels ("GPTQ, GPTAQ, and
//   RTN" wiki, quantizer; "ParoQuant" wiki, Straight-through estimation):
//     xmin = min(0, min x), xmax = max(0, max x)
//     symmetric: xmax = max(-xmin, xmax), xmin = -xmax when xmin < 0, zero = 8
//     all-zero range: [-1, 1]
//     scale = clamp((xmax - xmin) / 15, 1e-5, 1e5)
//     affine: zero = clamp(rne(-xmin / scale), 0, 15)
//     q = clamp(rne(x / scale) + zero, 0, 15)
//   stored: qweight [I][O/8] and qzeros [I/G][O/8] in AWQ nibble order,
//   scales [I/G][O] as fp16 (round to nearest even of the fp32 scale).
// Every decision is taken in fp32 with correctly rounded division.
//
// A workgroup (4 waves) takes one 128-channel block and 64 output rows; a
// wave takes 16 rows, rotates them in LDS with the activation path's staged
// code, reduces each row's range across the lanes of each G-group (G/2
// lanes), and quantizes.  Lane p holds input
// channels 2p, 2p+1 of all 16 rows, so it packs the qweight words of its two
// channels (8 rows each) without any exchange.
#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kQRS = kG + 4;  // LDS row stride (floats)

// AWQ word layout (awq_col in common.hpp): the slot holding column 8w + j
__device__ constexpr int awq_slot(int j) { return ((j & 1) << 2) | (j >> 1); }

template <int WDT>
__device__ __forceinline__ float2 load_w_pair(const void *w, int64_t idx) {
  if constexpr (WDT == kF32) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(w) + idx);
  } else {
    const uint32_t b = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(w) + idx);
    return float2{act_to_f32<WDT>(b & 0xffffu), act_to_f32<WDT>(b >> 16)};
  }
}

template <int WDT, bool SYM>
__global__ void __launch_bounds__(256)
quantize_pack_kernel(const void *__restrict__ w, int64_t O, int64_t I, const int16_t *__restrict__ pairs,
                     const float *__restrict__ theta, const float *__restrict__ cscale, int krot, int group,
                     int32_t *__restrict__ qweight, int32_t *__restrict__ qzeros, uint16_t *__restrict__ scales) {
  constexpr int RW = 16;
  __shared__ float lds[4][RW * kQRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * 64 + wave * RW;  // first output row of this wave
  if (n0 >= O) return;                                       // wave-uniform; no barriers below
  float *xs = lds[wave];

  const int gmask = kG - group;
  RotParams rp;
  rp.load(pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane, gmask);
  const float2 csv = *reinterpret_cast<const float2 *>(cscale + g * kG + 2 * lane);

  // W . D: the weight's input channels divided by the stored D^-1
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    float2 v{0.f, 0.f};
    if (n0 + m < O) v = load_w_pair<WDT>(w, (n0 + m) * I + g * kG + 2 * lane);
    xs[m * kQRS + 2 * lane] = v.x / csv.x;
    xs[m * kQRS + 2 * lane + 1] = v.y / csv.y;
  }
  wave_lds_sync();
  rotate_rows_lds<RW>(xs, kQRS, rp, pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane, gmask);

  // per row: range over the lanes of this lane's quantization group (G/2
  // lanes; zero included), parameters, codes
  uint32_t q0[RW], q1[RW];  // codes of channels 2p, 2p+1
  uint32_t zc[RW];
  float sc[RW];
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const float x0 = xs[m * kQRS + 2 * lane], x1 = xs[m * kQRS + 2 * lane + 1];
    float lo = fminf(fminf(x0, x1), 0.0f), hi = fmaxf(fmaxf(x0, x1), 0.0f);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      if (2 * d < group) {  // uniform: stays inside the G/2 lanes of the group
        lo = fminf(lo, __shfl_xor(lo, d));
        hi = fmaxf(hi, __shfl_xor(hi, d));
      }
    }
    if (SYM) {
      hi = fmaxf(-lo, hi);
      if (lo < 0.0f) lo = -hi;
    }
    if (lo == 0.0f && hi == 0.0f) {
      lo = -1.0f;
      hi = 1.0f;
    }
    float scale = (hi - lo) / 15.0f;
    scale = fminf(fmaxf(scale, 1e-5f), 1e5f);
    float zero = SYM ? 8.0f : fminf(fmaxf(__builtin_rintf(-lo / scale), 0.0f), 15.0f);
    q0[m] = (uint32_t)fminf(fmaxf(__builtin_rintf(x0 / scale) + zero, 0.0f), 15.0f);
    q1[m] = (uint32_t)fminf(fmaxf(__builtin_rintf(x1 / scale) + zero, 0.0f), 15.0f);
    zc[m] = (uint32_t)zero;
    sc[m] = scale;
  }

  // AWQ packing: column 8w+j of a word sits at nibble slot awq_slot(j).
  // This lane's quantization group (of I/G) and its index in that group.
  const int64_t qg = (g * kG + 2 * lane) / group;
  const int ql = (2 * lane) % group / 2;
  const int64_t W8 = O / 8;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t wcol = n0 / 8 + b;  // word column (8 output rows)
    if (n0 + 8 * b >= O) break;       // O % 8 == 0: a block of 8 rows is all in or all out
    uint32_t w0 = 0, w1 = 0, wz = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh = 4 * awq_slot(j);
      w0 |= q0[8 * b + j] << sh;
      w1 |= q1[8 * b + j] << sh;
      wz |= zc[8 * b + j] << sh;
    }
    const int64_t k = g * kG + 2 * lane;
    qweight[k * W8 + wcol] = (int32_t)w0;
    qweight[(k + 1) * W8 + wcol] = (int32_t)w1;
    if (ql == 0) qzeros[qg * W8 + wcol] = (int32_t)wz;  // the first lane of each group
  }
  // scales: lane ql < 16 of each group writes row n0 + ql of that group
  float my_scale = sc[0];
#pragma unroll
  for (int m = 1; m < RW; ++m)
    if (ql == m) my_scale = sc[m];
  if (ql < RW && n0 + ql < O) scales[qg * O + n0 + ql] = f32_to_f16_bits(my_scale);
}

template <int WDT>
static void launch_q(bool sym, dim3 grid, hipStream_t st, const void *w, int64_t O, int64_t I, const int16_t *pairs,
                     const float *theta, const float *cs, int krot, int group, int32_t *qw, int32_t *qz,
                     uint16_t *sc) {
  if (sym)
    hipLaunchKernelGGL((quantize_pack_kernel<WDT, true>), grid, dim3(256), 0, st, w, O, I, pairs, theta, cs, krot,
                       group, qw, qz, sc);
  else
    hipLaunchKernelGGL((quantize_pack_kernel<WDT, false>), grid, dim3(256), 0, st, w, O, I, pairs, theta, cs, krot,
                       group, qw, qz, sc);
}

hipError_t launch_quantize_pack(const void *w, int w_dt, bool sym, int64_t O, int64_t I, const int16_t *pairs,
                                const float *theta, const float *cs, int krot, int group, int32_t *qweight,
                                int32_t *qzeros, uint16_t *scales, hipStream_t st) {
  const dim3 grid((unsigned)(I / kG), (unsigned)((O + 63) / 64));
  if (w_dt == kF16)
    launch_q<kF16>(sym, grid, st, w, O, I, pairs, theta, cs, krot, group, qweight, qzeros, scales);
  else if (w_dt == kBF16)
    launch_q<kBF16>(sym, grid, st, w, O, I, pairs, theta, cs, krot, group, qweight, qzeros, scales);
  else
    launch_q<kF32>(sym, grid, st, w, O, I, pairs, theta, cs, krot, group, qweight, qzeros, scales);
  return hipGetLastError();
}

}  // namespace paro

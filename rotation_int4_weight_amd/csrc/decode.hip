// decode.hip - small-batch (tokens <= 16) rotated W4A16 linear: split-K MFMA
// GEMV, optionally with the activation rotation fused into the prologue.
//
//   y[m][n] = sum_g s[g][n] * sum_{k in g} x_r[m][k] * (q[k][n] - z[g][n]) + b[n]
//
// ("ParoQuant" wiki, Activation and weight transforms: Y = X_r Q(W_r)^T + b;
// Triton plans and tuning: unpack, subtract zero points, multiply by group
// scales, fp32 accumulation.)
//
// Work split.  A workgroup (4 waves) owns a tile of 128*WPL output columns
// and a range of `kgroups` 128-row groups; wave w takes groups w, w+4, ... of
// that range.  For one group a lane loads, for each of the group's four
// 32-row k-steps, the 8 rows of its 8-row block (lane>>4) of its WPL packed
// words (lane&15): a 16-lane row segment is contiguous in memory.  Each packed
// word turns into eight MFMA B fragments (one per nibble slot = one output
// column each), so no transpose is needed: v_perm_b32 gathers the bytes of a
// row pair and an OR with an exponent-bias constant turns a nibble into a
// half-precision number (fp16: 0x6400|q = 1024+q, 0x6400|(q<<4) = 1024+16q;
// bf16: 0x4300|q = 128+q).  The offset and the zero point are removed once per
// group, with the row sums of the rounded activations that one extra MFMA
// against a fragment of ones produces in the same output layout:
//   sum_k x (off + c*q) = off*xsum + c*sum_k x q
//   =>  sum_k x (q - z) = (acc - (off + c*z) * xsum) / c.
// v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A row l&15 and B column l&15 of
// its 8-element k block; the 16x16 fp32 result has row 4*(l>>4)+r, column
// l&15 in register r.
//
// Reduction.  The four waves' partial tiles are summed in LDS in wave order.
// With one K split the workgroup adds the bias and stores y.  Otherwise it
// stores its fp32 partial to the workspace, and the last workgroup of the
// column tile to arrive (device-scope counter) sums all partials in split
// order, adds the bias and stores y; it then resets the counter.  The result
// is therefore independent of arrival order (bitwise deterministic).
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kDecodeRS = kG + 4;  // fused-rotation LDS row stride (floats)

template <int DT>
struct MfmaTypes;
template <>
struct MfmaTypes<kF16> {
  typedef f16x8 v8;
  static constexpr uint32_t kMagic = 0x64006400u;  // 1024.0 in both halves
  static constexpr uint32_t kOnes = 0x3c003c00u;   // 1.0
  static constexpr float kOff = 1024.0f;
};
template <>
struct MfmaTypes<kBF16> {
  typedef bf16x8 v8;
  static constexpr uint32_t kMagic = 0x43004300u;  // 128.0 in both halves
  static constexpr uint32_t kOnes = 0x3f803f80u;   // 1.0
  static constexpr float kOff = 128.0f;
};

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  typedef typename MfmaTypes<DT>::v8 v8;
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0,
                                                   0, 0);
}

// B fragment of nibble slot `s` from the 8 row words r[0..7] (rows k0..k0+7)
// of one packed column word.  Element e of the fragment is row k0+e.
// fp16: even slots give 1024+q, odd slots 1024+16q; bf16: 128+q everywhere.
template <int DT>
__device__ __forceinline__ void build_b_frags(const uint32_t r[8], u32x4 out[8]) {
  constexpr uint32_t M = MfmaTypes<DT>::kMagic;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // P = [ra.b0, ra.b2, rb.b0, rb.b2], Q = [ra.b1, ra.b3, rb.b1, rb.b3]
    const uint32_t P = __builtin_amdgcn_perm(r[2 * i], r[2 * i + 1], 0x02000604u);
    const uint32_t Q = __builtin_amdgcn_perm(r[2 * i], r[2 * i + 1], 0x03010705u);
    const uint32_t P8 = P >> 8, Q8 = Q >> 8;
    if constexpr (DT == kF16) {
      out[0][i] = (P & 0x000f000fu) | M;
      out[1][i] = (P & 0x00f000f0u) | M;
      out[2][i] = (Q & 0x000f000fu) | M;
      out[3][i] = (Q & 0x00f000f0u) | M;
      out[4][i] = (P8 & 0x000f000fu) | M;
      out[5][i] = (P8 & 0x00f000f0u) | M;
      out[6][i] = (Q8 & 0x000f000fu) | M;
      out[7][i] = (Q8 & 0x00f000f0u) | M;
    } else {
      out[0][i] = (P & 0x000f000fu) | M;
      out[1][i] = ((P >> 4) & 0x000f000fu) | M;
      out[2][i] = (Q & 0x000f000fu) | M;
      out[3][i] = ((Q >> 4) & 0x000f000fu) | M;
      out[4][i] = (P8 & 0x000f000fu) | M;
      out[5][i] = ((P >> 12) & 0x000f000fu) | M;
      out[6][i] = (Q8 & 0x000f000fu) | M;
      out[7][i] = ((Q >> 12) & 0x000f000fu) | M;
    }
  }
}

// Scale factor c of slot s in the fragment encoding (see build_b_frags).
template <int DT>
__device__ __forceinline__ constexpr float slot_mult(int s) {
  return (DT == kF16 && (s & 1)) ? 16.0f : 1.0f;
}

template <int DT, int WPL, bool FUSED, int FR>
__global__ void __launch_bounds__(256)
decode_kernel(LinearArgs a, const uint16_t *__restrict__ xr, int kgroups, int splits,
              float *__restrict__ partial, uint32_t *__restrict__ counters) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_last;
  const int lane = lane_id(), wave = wave_id();
  const int cl = lane & 15, kb = lane >> 4;
  const int ntile = 128 * WPL;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int64_t I = a.I, O = a.O, W = O / 8;
  const int M = (int)a.tokens;
  const int64_t ngroups = I / kG;
  const int64_t g_begin = (int64_t)split * kgroups;
  const int64_t g_end = (g_begin + kgroups < ngroups) ? g_begin + kgroups : ngroups;
  const int64_t word_base = (int64_t)tile * 16 * WPL + cl * WPL;  // this lane's first word
  const uint16_t *__restrict__ x = reinterpret_cast<const uint16_t *>(a.x);

  f32x4 tot[WPL * 8];
#pragma unroll
  for (int j = 0; j < WPL * 8; ++j) tot[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  float *xs = smem + wave * (16 * kDecodeRS);  // fused rotation rows of this wave

  for (int64_t g = g_begin + wave; g < g_end; g += 4) {
    // ---- issue the group's weight loads first (they dominate latency) ----
    uint32_t qv[4][8][WPL];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t k = g * kG + ks * 32 + kb * 8 + r;
        const int32_t *row = a.qweight + k * W;
#pragma unroll
        for (int w = 0; w < WPL; ++w) {
          const int64_t wi = word_base + w;
          qv[ks][r][w] = (wi < W) ? (uint32_t)row[wi] : 0u;
        }
      }
    }
    u32x4 sv[WPL];
    uint32_t zv[WPL];
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      const int64_t wi = word_base + w;
      if (wi < W) {
        sv[w] = *reinterpret_cast<const u32x4 *>(a.scales + g * O + 8 * wi);
        zv[w] = (uint32_t)a.qzeros[g * W + wi];
      } else {
        sv[w] = u32x4{0u, 0u, 0u, 0u};
        zv[w] = 0u;
      }
    }

    // ---- A fragments: rotated activations of this group, rounded to DT ----
    u32x4 af[4];
    if constexpr (FUSED) {
      const int64_t c0 = g * kG + 2 * lane;
      const float s0 = a.cs[c0], s1 = a.cs[c0 + 1];
      for (int m = 0; m < M; ++m) {
        const uint32_t wv = *reinterpret_cast<const uint32_t *>(x + (int64_t)m * I + c0);
        xs[m * kDecodeRS + 2 * lane] = act_to_f32<DT>(wv & 0xffffu) * s0;
        xs[m * kDecodeRS + 2 * lane + 1] = act_to_f32<DT>(wv >> 16) * s1;
      }
      wave_lds_sync();
      rotate_rows_lds<16>(xs, kDecodeRS, M, a.pairs + g * kG, I, a.theta + g * kPairs, I / 2, a.krot, lane);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (cl < M) {
          const float *src = xs + cl * kDecodeRS + ks * 32 + kb * 8;
          const float4 lo = *reinterpret_cast<const float4 *>(src);
          const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
          af[ks] = u32x4{pack2<DT>(lo.x, lo.y), pack2<DT>(lo.z, lo.w), pack2<DT>(hi.x, hi.y),
                         pack2<DT>(hi.z, hi.w)};
        } else {
          af[ks] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      wave_lds_sync();  // the next group's rotation rewrites xs
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        af[ks] = (cl < M) ? *reinterpret_cast<const u32x4 *>(xr + (int64_t)cl * I + g * kG + ks * 32 + kb * 8)
                          : u32x4{0u, 0u, 0u, 0u};
      }
    }

    // ---- row sums of the rounded activations (same layout as the output) ----
    const u32x4 ones = {MfmaTypes<DT>::kOnes, MfmaTypes<DT>::kOnes, MfmaTypes<DT>::kOnes,
                        MfmaTypes<DT>::kOnes};
    f32x4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) xsum = mfma16<DT>(af[ks], ones, xsum);

    // ---- the group's products ----
    f32x4 acc[WPL * 8];
#pragma unroll
    for (int j = 0; j < WPL * 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        uint32_t rw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) rw[r] = qv[ks][r][w];
        u32x4 bf[8];
        build_b_frags<DT>(rw, bf);
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[w * 8 + s] = mfma16<DT>(af[ks], bf[s], acc[w * 8 + s]);
      }
    }

    // ---- fold: tot += s/c * (acc - (off + c*z) * xsum) ----
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int col = awq_col(s);
        const uint32_t sb = (sv[w][col >> 1] >> (16 * (col & 1))) & 0xffffu;
        const float c = slot_mult<DT>(s);
        const float sc = f16_bits_to_f32(sb) * (1.0f / c);
        const float zz = MfmaTypes<DT>::kOff + c * (float)((zv[w] >> (4 * s)) & 0xfu);
#pragma unroll
        for (int i = 0; i < FR; ++i) tot[w * 8 + s][i] += sc * (acc[w * 8 + s][i] - zz * xsum[i]);
      }
    }
  }

  // ---- reduce the four waves' tiles in LDS (wave order) ----
  const int rows = (FR < 4) ? FR : 16;  // rows held in registers across the wave
  __syncthreads();  // every wave is done with its rotation rows
  float *red = smem;  // [4][rows][ntile]
#pragma unroll
  for (int w = 0; w < WPL; ++w) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int col = (cl * WPL + w) * 8 + awq_col(s);
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int row = 4 * kb + i;
        if (row < rows) red[(wave * rows + row) * ntile + col] = tot[w * 8 + s][i];
      }
    }
  }
  __syncthreads();

  const int64_t n0 = (int64_t)tile * ntile;
  const int nel = M * ntile;
  const bool direct = (splits == 1);
  for (int e = threadIdx.x; e < nel; e += 256) {
    const int row = e / ntile, col = e - row * ntile;
    const float v = ((red[(0 * rows + row) * ntile + col] + red[(1 * rows + row) * ntile + col]) +
                     red[(2 * rows + row) * ntile + col]) +
                    red[(3 * rows + row) * ntile + col];
    const int64_t n = n0 + col;
    if (n >= O) continue;
    if (direct) {
      const float out = v + (a.bias ? f16_bits_to_f32(a.bias[n]) : 0.0f);
      if (a.y_dt == kF32) reinterpret_cast<float *>(a.y)[(int64_t)row * O + n] = out;
      else if (a.y_dt == kF16) reinterpret_cast<uint16_t *>(a.y)[(int64_t)row * O + n] = f32_to_f16_bits(out);
      else reinterpret_cast<uint16_t *>(a.y)[(int64_t)row * O + n] = f32_to_bf16_bits(out);
    } else {
      partial[((int64_t)split * M + row) * O + n] = v;
    }
  }
  if (direct) return;

  __threadfence();  // release this workgroup's partial (device scope)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&counters[tile], 1u);
    s_last = (old == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire every other workgroup's partial
  for (int e = threadIdx.x; e < nel; e += 256) {
    const int row = e / ntile, col = e - row * ntile;
    const int64_t n = n0 + col;
    if (n >= O) continue;
    float v = 0.0f;
    for (int sp = 0; sp < splits; ++sp) v += __builtin_nontemporal_load(&partial[((int64_t)sp * M + row) * O + n]);
    const float out = v + (a.bias ? f16_bits_to_f32(a.bias[n]) : 0.0f);
    if (a.y_dt == kF32) reinterpret_cast<float *>(a.y)[(int64_t)row * O + n] = out;
    else if (a.y_dt == kF16) reinterpret_cast<uint16_t *>(a.y)[(int64_t)row * O + n] = f32_to_f16_bits(out);
    else reinterpret_cast<uint16_t *>(a.y)[(int64_t)row * O + n] = f32_to_bf16_bits(out);
  }
  if (threadIdx.x == 0) atomicExch(&counters[tile], 0u);
}

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

DecodePlan plan_decode(int64_t I, int64_t O, int64_t tokens, bool fused) {
  (void)fused;
  DecodePlan p;
  p.wpl = 1;
  p.ntile = 128 * p.wpl;
  p.n_tiles = (int)((O + p.ntile - 1) / p.ntile);
  const int64_t ngroups = I / kG;
  // Largest multiple of 4 groups per workgroup that still fills the chip
  // with one full wave of workgroups; fewer K splits mean less partial-sum
  // traffic (tokens * O * 4 bytes written and read per extra split).
  int kg = 4;
  for (int cand = 4; cand <= 4 * ((ngroups + 3) / 4); cand *= 2) {
    const int64_t wgs = (int64_t)p.n_tiles * ((ngroups + cand - 1) / cand);
    if (wgs >= 240) kg = cand;
  }
  const int forced = env_int("PARO_DECODE_KGROUPS", 0);
  if (forced > 0) kg = forced;
  (void)tokens;
  p.kgroups = kg;
  p.splits = (int)((ngroups + kg - 1) / kg);
  return p;
}

size_t decode_partial_bytes(const DecodePlan &p, int64_t tokens, int64_t O) {
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * (size_t)tokens * (size_t)O * 4;
}

template <int DT, int WPL, bool FUSED>
static hipError_t launch_decode_t(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                                  float *partial, hipStream_t st) {
  dim3 grid((unsigned)p.n_tiles, (unsigned)p.splits);
  const int M = (int)a.tokens;
  const int rows = (M <= 1) ? 1 : (M <= 2) ? 2 : 16;
  size_t red_bytes = (size_t)4 * rows * p.ntile * 4;
  size_t rot_bytes = FUSED ? (size_t)4 * 16 * kDecodeRS * 4 : 0;
  size_t shmem = red_bytes > rot_bytes ? red_bytes : rot_bytes;
  const uint16_t *xrp = reinterpret_cast<const uint16_t *>(xr);
  if (M <= 1)
    hipLaunchKernelGGL((decode_kernel<DT, WPL, FUSED, 1>), grid, dim3(256), shmem, st, a, xrp, p.kgroups,
                       p.splits, partial, counters);
  else if (M <= 2)
    hipLaunchKernelGGL((decode_kernel<DT, WPL, FUSED, 2>), grid, dim3(256), shmem, st, a, xrp, p.kgroups,
                       p.splits, partial, counters);
  else
    hipLaunchKernelGGL((decode_kernel<DT, WPL, FUSED, 4>), grid, dim3(256), shmem, st, a, xrp, p.kgroups,
                       p.splits, partial, counters);
  return hipGetLastError();
}

hipError_t launch_decode(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                         float *partials, hipStream_t st) {
  const bool fused = (xr == nullptr);
#define PARO_DECODE_CASE(DT, WPL)                                                   \
  return fused ? launch_decode_t<DT, WPL, true>(a, p, xr, counters, partials, st) \
               : launch_decode_t<DT, WPL, false>(a, p, xr, counters, partials, st)
  if (a.x_dt == kF16) {
    if (p.wpl == 2) PARO_DECODE_CASE(kF16, 2);
    PARO_DECODE_CASE(kF16, 1);
  }
  if (p.wpl == 2) PARO_DECODE_CASE(kBF16, 2);
  PARO_DECODE_CASE(kBF16, 1);
#undef PARO_DECODE_CASE
}

}  // namespace paro

// decode.hip - small-batch (tokens <= 16) rotated W4A16 linear: split-K MFMA
// GEMV, optionally with the activation rotation fused into the prologue.
//
//   y[m][n] = sum_g s[g][n] * sum_{k in g} x_r[m][k] * (q[k][n] - z[g][n]) + b[n]
//
// ("ParoQuant" wiki, Activation and weight transforms: Y = X_r Q(W_r)^T + b;
// Triton plans and tuning: unpack, subtract zero points, multiply by group
// scales, fp32 accumulation.)
//
// Work split.  A k-step is 32 rows of the weight.  A workgroup (NW waves)
// owns a tile of 128*WPL output columns and NW*KSW consecutive k-steps; wave
// w takes KSW consecutive k-steps of them.  For one k-step a lane loads the 8 rows of
// its 8-row block (lane>>4) of its WPL consecutive packed words (lane&15), so
// the 16 lanes of a block read 64*WPL contiguous bytes of each row (256 B
// with WPL = 4).  A wave issues the loads of all its k-steps before it
// computes, in the order it consumes them, so the MFMAs of a k-step start as
// soon as its own loads have landed.  Each packed word turns into eight MFMA
// B fragments (one per nibble slot = one output column each), so no
// transpose is needed: v_perm_b32 gathers the bytes of a row pair and an OR
// with an exponent-bias constant turns a nibble into a half-precision number
// (fp16: 0x6400|q = 1024+q, 0x6400|(q<<4) = 1024+16q; bf16: 0x4300|q =
// 128+q).  The offset and the zero point are removed with the row sums of the
// rounded activations, which one extra MFMA against a fragment of ones
// produces in the output layout:
//   sum_k x (off + c*q) = off*xsum + c*sum_k x q
//   =>  sum_k x (q - z) = (acc - (off + c*z) * xsum) / c,
// folded into the running sum with the group scale once per group (or per
// k-step when a wave owns a single k-step; the fold is linear, so both are the
// same sum).  v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A row l&15 and B
// column l&15 of its 8-element k block; the 16x16 fp32 result has row
// 4*(l>>4)+r, column l&15 in register r.
//
// Workgroups are numbered tile-fastest (all column tiles of split 0, then of
// split 1, ...) and that order is dealt out to the XCDs in contiguous runs
// (xcd_local_order), so the tiles sharing the same weight rows run on one XCD
// at the same time and their row segments merge in its L2 into long DRAM
// bursts.
//
// Reduction.  The NW waves' tiles are summed in LDS in wave order, each
// thread taking quads of 4 consecutive outputs.  With one K split the
// workgroup adds the bias and stores y.  Otherwise it stores its fp32 partial
// with 16-byte device-coherent stores (SC1: coherent across the XCDs' L2
// caches without whole-cache write-backs), waits for them, and bumps a
// device-scope counter; the last workgroup of the column tile to arrive
// loads every split's quads with 16-byte device-coherent loads, all in flight
// together, sums them in split order, adds the bias, stores y and resets the
// counter.  The result is independent of arrival order (bitwise
// deterministic).
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kDecodeRS = kG + 4;  // fused-rotation LDS row stride (floats)
constexpr int kCounterStride = 32; // uint32 per split-K counter: one 128-byte line each
// Cache policy of the raw buffer loads/stores that exchange split-K partials:
// SC1, the device-scope coherent form (the one relaxed device-scope atomics use).
constexpr int kDeviceCoherent = 16;

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

// Load WPL consecutive packed words of one row (one vector load when WPL > 1).
template <int WPL>
__device__ __forceinline__ void load_words(const int32_t *__restrict__ p, uint32_t out[WPL]) {
  if constexpr (WPL == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else if constexpr (WPL == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
    out[0] = v[0]; out[1] = v[1];
  } else {
    out[0] = (uint32_t)p[0];
  }
}

// MT: token rows carried per wave (1, 2, 4, 8 or 16; M <= MT, rows >= M are
// zero).  FR = min(MT, 4) accumulator registers can hold real rows.
template <int DT, int WPL, int KSW, int NW, bool FUSED, int MT>
__global__ void __launch_bounds__(64 * NW)
decode_kernel(LinearArgs a, const uint16_t *__restrict__ xr, int splits, float *__restrict__ partial,
              uint32_t *__restrict__ counters) {
  constexpr int FR = MT < 4 ? MT : 4;
  constexpr int NT = 8 * WPL;                 // MFMA column tiles per wave
  constexpr int NG = KSW < 4 ? 1 : KSW / 4;   // groups a wave touches (its k-steps are aligned)
  // k-steps of loads kept in flight (16-wave groups have half the registers)
  constexpr int PD = KSW < (NW >= 16 ? 2 : 4) ? KSW : (NW >= 16 ? 2 : 4);
  constexpr int NTH = 64 * NW;
  constexpr int NTILE = 128 * WPL;
  constexpr int QUADS = MT * NTILE / 4;                 // 4-column output quads of the tile
  constexpr int QPT = (QUADS + NTH - 1) / NTH;          // quads per thread
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_last;
  const int lane = lane_id(), wave = wave_id();
  const int cl = lane & 15, kb = lane >> 4;
  const int n_tiles = (int)((a.O + NTILE - 1) / NTILE);
  const int lwg = xcd_local_order((int)blockIdx.x, n_tiles * splits);
  const int tile = lwg % n_tiles, split = lwg / n_tiles;
  const int64_t I = a.I, O = a.O, W = O / 8;
  const int M = (int)a.tokens;
  const int64_t nks = I / 32;
  const int64_t ks0 = ((int64_t)split * NW + wave) * KSW;  // first k-step of this wave
  const int nk = (int)((ks0 >= nks) ? 0 : ((nks - ks0) < KSW ? (nks - ks0) : KSW));
  const uint16_t *__restrict__ x = reinterpret_cast<const uint16_t *>(a.x);
  const int64_t n0 = (int64_t)tile * NTILE;

  // ---- small early loads: this thread's bias values ----
  // Quad q holds outputs 4q..4q+3 of the tile ([row][col], NTILE columns per
  // row); a quad is entirely inside or entirely past O (O % 8 == 0).
  // Branch-free: every load reads a valid address (a stand-in tensor when
  // there is no bias, a clamped column past O) and the value is selected
  // afterwards.  A conditional load would make the compiler wait for it at
  // the join, i.e. one full memory round trip before the weight stream.
  float bias_v[QPT][4];
  const uint16_t *bias_src = a.bias ? a.bias : a.scales;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int q = threadIdx.x + j * NTH;
    const int64_t n = n0 + (4 * q) % NTILE;
    const bool use = a.bias && q < M * NTILE / 4 && n < O;
    const u32x2 b = *reinterpret_cast<const u32x2 *>(bias_src + (n < O ? n : O - 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) bias_v[j][c] = use ? f16_bits_to_f32((b[c >> 1] >> (16 * (c & 1))) & 0xffffu) : 0.0f;
  }

  // Columns past O (last tile only) read an in-bounds word and are zeroed;
  // their outputs are never stored.  WPL words never straddle O (O % 16 == 0
  // for WPL == 2, O % 32 == 0 for WPL == 4).
  const int64_t wbase = (int64_t)tile * 16 * WPL + cl * WPL;
  const bool wok = wbase < W;
  const int64_t wcl = wok ? wbase : W - WPL;

  float tot[NT][FR];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < FR; ++i) tot[j][i] = 0.0f;

  if (nk > 0) {
    // 128-channel rotation blocks hold 4 k-steps; quantization groups hold
    // G/32 = 1 << gsh (with G < 128 the plan gives each wave one k-step)
    const int gsh = __builtin_ctz((unsigned)a.group) - 5, gmask = kG - a.group;
    const int64_t g_first = ks0 / 4, q_first = ks0 >> gsh, nq = I / a.group;
    float *xs = smem + wave * (MT * kDecodeRS);  // fused rotation rows of this wave
    // ---- fused: the first group's rotation inputs, before the weight stream ----
    RotParams rp;
    float xin[MT][2];
    float cs0 = 0.f, cs1 = 0.f;
    auto load_rot_inputs = [&](int64_t g) {
      const int64_t c0 = g * kG + 2 * lane;
      rp.load(a.pairs + g * kG, I, a.theta + g * kPairs, I / 2, a.krot, lane, gmask);
      cs0 = a.cs[c0];
      cs1 = a.cs[c0 + 1];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t wv = *reinterpret_cast<const uint32_t *>(x + (int64_t)(m < M ? m : 0) * I + c0);
        xin[m][0] = act_to_f32<DT>(wv & 0xffffu);
        xin[m][1] = act_to_f32<DT>(wv >> 16);
      }
    };
    if constexpr (FUSED) load_rot_inputs(g_first);

    // ---- A fragments (non-fused), group scales / zeros, then the weights of
    //      the first PD k-steps, in the order they are consumed ----
    u32x4 af[KSW];
    const int arow = cl < M ? cl : 0;
    auto load_a = [&](int k) {  // non-fused: rotated activations from the workspace
      const int64_t ks = ks0 + (k < nk ? k : 0);
      af[k] = *reinterpret_cast<const u32x4 *>(xr + (int64_t)arow * I + ks * 32 + kb * 8);
      if (cl >= M) af[k] = u32x4{0u, 0u, 0u, 0u};
    };
    if constexpr (!FUSED) {
#pragma unroll
      for (int k = 0; k < PD; ++k) load_a(k);
    }
    u32x4 sv[NG][WPL];
    uint32_t zv[NG][WPL];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int64_t g0 = q_first + gi;
      const int64_t g = g0 < nq ? g0 : nq - 1;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        sv[gi][w] = *reinterpret_cast<const u32x4 *>(a.scales + g * O + 8 * (wcl + w));  // wcl is in bounds
        if (!wok) sv[gi][w] = u32x4{0u, 0u, 0u, 0u};
        zv[gi][w] = (uint32_t)a.qzeros[g * W + wcl + w];
      }
    }
    uint32_t qv[KSW][8][WPL];
    auto load_ks = [&](int k) {
      const int64_t ks = ks0 + (k < nk ? k : 0);
#pragma unroll
      for (int r = 0; r < 8; ++r) load_words<WPL>(a.qweight + (ks * 32 + kb * 8 + r) * W + wcl, qv[k][r]);
    };
#pragma unroll
    for (int k = 0; k < PD; ++k) load_ks(k);

    const u32x4 ones = {MfmaTypes<DT>::kOnes, MfmaTypes<DT>::kOnes, MfmaTypes<DT>::kOnes,
                        MfmaTypes<DT>::kOnes};
    f32x4 acc[NT];
    f32x4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int k = 0; k < KSW; ++k) {
      if (k < nk) {
        const int64_t ks = ks0 + k;
        const int64_t g = ks / 4;                     // rotation block
        const int gi = (int)((ks >> gsh) - q_first);  // quantization group of this wave
        if constexpr (FUSED) {
          if (k == 0 || (ks % 4) == 0) {  // entering a group: rotate it into LDS
            if (k != 0) load_rot_inputs(g);
            wave_lds_sync();
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              xs[m * kDecodeRS + 2 * lane] = m < M ? xin[m][0] * cs0 : 0.0f;
              xs[m * kDecodeRS + 2 * lane + 1] = m < M ? xin[m][1] * cs1 : 0.0f;
            }
            wave_lds_sync();
            rotate_rows_lds<MT>(xs, kDecodeRS, rp, a.pairs + g * kG, I, a.theta + g * kPairs, I / 2, a.krot,
                                lane, gmask);
          }
          const float *src = xs + (cl < MT ? cl : 0) * kDecodeRS + (ks % 4) * 32 + kb * 8;
          const float4 lo = *reinterpret_cast<const float4 *>(src);
          const float4 hi = *reinterpret_cast<const float4 *>(src + 4);
          af[k] = u32x4{pack2<DT>(lo.x, lo.y), pack2<DT>(lo.z, lo.w), pack2<DT>(hi.x, hi.y),
                        pack2<DT>(hi.z, hi.w)};
          if (cl >= M) af[k] = u32x4{0u, 0u, 0u, 0u};
        }
        if (k + PD < KSW) {  // keep PD k-steps in flight
          if constexpr (!FUSED) load_a(k + PD);
          load_ks(k + PD);
        }
        xsum = mfma16<DT>(af[k], ones, xsum);
#pragma unroll
        for (int w = 0; w < WPL; ++w) {
          uint32_t rw[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) rw[r] = qv[k][r][w];
          u32x4 bf[8];
          build_b_frags<DT>(rw, bf);
#pragma unroll
          for (int s = 0; s < 8; ++s) acc[w * 8 + s] = mfma16<DT>(af[k], bf[s], acc[w * 8 + s]);
        }
        // fold at the end of a group or of this wave's k-steps:
        //   tot += s/c * (acc - (off + c*z) * xsum)
        if (((ks + 1) & ((1 << gsh) - 1)) == 0 || k == nk - 1) {
#pragma unroll
          for (int w = 0; w < WPL; ++w) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int col = awq_col(s);
              const uint32_t sb = (sv[gi][w][col >> 1] >> (16 * (col & 1))) & 0xffffu;
              const float c = slot_mult<DT>(s);
              const float sc = f16_bits_to_f32(sb) * (1.0f / c);
              const float zz = MfmaTypes<DT>::kOff + c * (float)((zv[gi][w] >> (4 * s)) & 0xfu);
#pragma unroll
              for (int i = 0; i < FR; ++i) tot[w * 8 + s][i] += sc * (acc[w * 8 + s][i] - zz * xsum[i]);
              acc[w * 8 + s] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
          xsum = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }

  // ---- reduce the NW waves' tiles in LDS (wave order) ----
  __syncthreads();   // every wave is done with its rotation rows
  float *red = smem; // [NW][MT][NTILE]
#pragma unroll
  for (int w = 0; w < WPL; ++w) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int col = (cl * WPL + w) * 8 + awq_col(s);
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int row = 4 * kb + i;
        if (row < MT) red[(wave * MT + row) * NTILE + col] = tot[w * 8 + s][i];
      }
    }
  }
  __syncthreads();

  // quads of this thread: sum over the waves in wave order
  const int nq = M * NTILE / 4;  // quads holding real rows
  f32x4 v[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int q = threadIdx.x + j * NTH;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (q < nq) {
#pragma unroll
      for (int w = 0; w < NW; ++w) v[j] += *reinterpret_cast<const f32x4 *>(red + w * MT * NTILE + 4 * q);
    }
  }
  auto quad_out = [&](int j, int &row, int64_t &n) {
    const int q = threadIdx.x + j * NTH;
    row = (4 * q) / NTILE;
    n = n0 + (4 * q - row * NTILE);
    return q < nq && n < O;
  };
  auto store_quads = [&](const f32x4 *val) {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      int row;
      int64_t n;
      if (quad_out(j, row, n)) {
        const float o0 = val[j][0] + bias_v[j][0], o1 = val[j][1] + bias_v[j][1];
        const float o2 = val[j][2] + bias_v[j][2], o3 = val[j][3] + bias_v[j][3];
        if (a.y_dt == kF32) {
          *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.y) + row * O + n) = f32x4{o0, o1, o2, o3};
        } else {
          u32x2 h;
          if (a.y_dt == kF16) h = u32x2{pack2<kF16>(o0, o1), pack2<kF16>(o2, o3)};
          else h = u32x2{pack2<kBF16>(o0, o1), pack2<kBF16>(o2, o3)};
          *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.y) + row * O + n) = h;
        }
      }
    }
  };
  if (splits == 1) {
    store_quads(v);
    return;
  }

  // ---- split-K handoff (see the header) ----
  // partial: [tile][split][M][NTILE] fp32.  One raw buffer per tile: its
  // splits * M * NTILE * 4 bytes (at most 2^14 * 16 * 512 * 4 = 2^29) keep
  // every offset in 32 bits.
  const uint32_t sstride = (uint32_t)(M * NTILE);  // floats per split
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      partial + (int64_t)tile * splits * sstride, (short)0, (int)((uint32_t)splits * sstride * 4u), 0x00020000);
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    int row;
    int64_t n;
    if (quad_out(j, row, n))
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[j]), prs,
                                             ((uint32_t)split * sstride + 4u * (uint32_t)(threadIdx.x + j * NTH)) * 4u,
                                             0, kDeviceCoherent);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  uint32_t *cnt = counters + (int64_t)tile * kCounterStride;
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (uint32_t)(splits - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // Gather every split's quads, all loads of a batch in flight together (the
  // addresses of splits past the last are clamped and their values dropped),
  // summing in split order.
  constexpr int SB = QPT >= 16 ? 1 : 16 / QPT;  // splits per batch
  f32x4 sum[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) sum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; sp += SB) {
    f32x4 t[QPT][SB];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const uint32_t q = (uint32_t)(threadIdx.x + j * NTH);
      const uint32_t off = 16u * (q < (uint32_t)nq ? q : 0u);
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const uint32_t spc = (uint32_t)(sp + u < splits ? sp + u : splits - 1);
        t[j][u] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, off + spc * sstride * 4u, 0, kDeviceCoherent));
      }
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j)
#pragma unroll
      for (int u = 0; u < SB; ++u)
        if (sp + u < splits) sum[j] += t[j][u];
  }
  store_quads(sum);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

DecodePlan plan_decode(int64_t I, int64_t O, int64_t tokens, bool fused, int group) {
  (void)fused;
  DecodePlan p;
  const int64_t nks = I / 32;
  if (tokens <= 4) {
    // Few rows: the per-k-step fold is nearly free (one register row), so a
    // wave owns one k-step of 128-byte row segments; eight waves per
    // workgroup keep the K splits (whose partials the last workgroup gathers)
    // at nks / 8 while filling the chip.
    p.wpl = (O % 16 == 0) ? 2 : 1;
    p.ksw = 1;
    p.nw = 8;
  } else {
    // Up to 16 rows: the partial sums cost splits * tokens * O * 8 bytes, so
    // an eight-wave workgroup covers long K ranges (several k-steps per wave,
    // folded once per group).  256-column tiles with four k-steps per wave
    // measured fastest on 4096 -> 14336 at 16 tokens (one 128-byte segment
    // per weight row and lane group, four splits).
    p.wpl = (O % 16 == 0) ? 2 : 1;
    p.nw = 8;
    p.ksw = p.wpl == 2 ? 4 : 8;
    while (p.ksw > 1 && (int64_t)p.nw * (p.ksw / 2) >= nks) p.ksw /= 2;
  }
  // Tuning overrides, read once per process: PARO_DECODE_WPL / _KSW / _NW.
  static const int fw = env_int("PARO_DECODE_WPL", 0);
  static const int fk = env_int("PARO_DECODE_KSW", 0);
  static const int fn = env_int("PARO_DECODE_NW", 0);
  if (fw == 1 || (fw == 2 && O % 16 == 0) || (fw == 4 && O % 32 == 0)) p.wpl = fw;
  if (fk == 1 || fk == 2 || fk == 4 || fk == 8) p.ksw = fk;
  if (fn == 4 || fn == 8 || fn == 16) p.nw = fn;
  // groups of 32 or 64 rows: one k-step per wave (the kernel keeps one
  // group's scales and zeros per wave and folds every k-step)
  if (group < kG) p.ksw = 1;
  p.ntile = 128 * p.wpl;
  p.n_tiles = (int)((O + p.ntile - 1) / p.ntile);
  p.splits = (int)((nks + p.nw * p.ksw - 1) / (p.nw * p.ksw));
  return p;
}

size_t decode_partial_bytes(const DecodePlan &p, int64_t tokens, int64_t O) {
  (void)O;
  if (p.splits <= 1) return 0;
  // [tile][split][tokens][ntile] fp32
  return (size_t)p.n_tiles * (size_t)p.splits * (size_t)tokens * (size_t)p.ntile * 4;
}

template <int DT, int WPL, int KSW, int NW, bool FUSED>
static hipError_t launch_decode_t(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                                  float *partial, hipStream_t st) {
  dim3 grid((unsigned)(p.n_tiles * p.splits));
  const int M = (int)a.tokens;
  const int mt = (M <= 1) ? 1 : (M <= 2) ? 2 : (M <= 4) ? 4 : (M <= 8) ? 8 : 16;
  size_t red_bytes = (size_t)NW * mt * p.ntile * 4;
  size_t rot_bytes = FUSED ? (size_t)NW * mt * kDecodeRS * 4 : 0;
  size_t shmem = red_bytes > rot_bytes ? red_bytes : rot_bytes;
  const uint16_t *xrp = reinterpret_cast<const uint16_t *>(xr);
#define PARO_DECODE_LAUNCH(MT)                                                                                \
  hipLaunchKernelGGL((decode_kernel<DT, WPL, KSW, NW, FUSED, MT>), grid, dim3(64 * NW), shmem, st, a, xrp, p.splits, \
                     partial, counters)
  switch (mt) {
    case 1: PARO_DECODE_LAUNCH(1); break;
    case 2: PARO_DECODE_LAUNCH(2); break;
    case 4: PARO_DECODE_LAUNCH(4); break;
    case 8: PARO_DECODE_LAUNCH(8); break;
    default: PARO_DECODE_LAUNCH(16); break;
  }
#undef PARO_DECODE_LAUNCH
  return hipGetLastError();
}

template <int DT, bool FUSED>
static hipError_t launch_decode_dt(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                                   float *partials, hipStream_t st) {
  // every (wpl, ksw, nw) the planner produces is instantiated; other
  // combinations (tuning overrides only) are rejected
#define PARO_DECODE_CFG(WPL, KSW, NW) \
  if (p.wpl == WPL && p.ksw == KSW && p.nw == NW) return launch_decode_t<DT, WPL, KSW, NW, FUSED>(a, p, xr, counters, partials, st)
  PARO_DECODE_CFG(2, 1, 8);
  PARO_DECODE_CFG(1, 1, 8);
  PARO_DECODE_CFG(2, 1, 16);
  PARO_DECODE_CFG(4, 1, 8);
  PARO_DECODE_CFG(2, 2, 4);
  PARO_DECODE_CFG(1, 8, 16);
  PARO_DECODE_CFG(1, 8, 8);
  PARO_DECODE_CFG(1, 4, 8);
  PARO_DECODE_CFG(1, 2, 8);
  PARO_DECODE_CFG(2, 4, 8);
  PARO_DECODE_CFG(2, 2, 8);
  PARO_DECODE_CFG(1, 4, 16);
  PARO_DECODE_CFG(1, 2, 16);
  PARO_DECODE_CFG(1, 1, 16);
  PARO_DECODE_CFG(1, 8, 4);
  PARO_DECODE_CFG(1, 4, 4);
#undef PARO_DECODE_CFG
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                         float *partials, hipStream_t st) {
  const bool fused = (xr == nullptr);
  if (a.x_dt == kF16)
    return fused ? launch_decode_dt<kF16, true>(a, p, xr, counters, partials, st)
                 : launch_decode_dt<kF16, false>(a, p, xr, counters, partials, st);
  return fused ? launch_decode_dt<kBF16, true>(a, p, xr, counters, partials, st)
               : launch_decode_dt<kBF16, false>(a, p, xr, counters, partials, st);
}

}  // namespace paro

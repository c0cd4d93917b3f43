// rotate_backward.hip - backward of the channel scaling and pairwise rotation
// (the calibration step of the method: the optimizer updates angles and
// channel scales through the rotation; "ParoQuant" wiki, Straight-through
// estimation, and the pair formula of Concepts / Pairwise Givens rotations).
//
// Per 128-channel group, x_r = y_K with y_0 = x * cs and y_t = y_{t-1} . R_t,
// where R_t is stage t's set of Givens rotations (a' = a c + b s,
// b' = -a s + b c).  For g = dL/dx_r, gy_t = g . (R_{t+1} ... R_K)^T, and
//   dL/dtheta_t(p) = sum over tokens of ga' b' - gb' a' = N_t[a][b] - N_t[b][a]
// with N_t = gy_t^T . y_t, a 128 x 128 matrix per group.  Since the stages are
// orthogonal, N_t = R_t^T N_{t-1} R_t and N_0 = R . C . diag(cs) with
// R = R_1 ... R_K and the Gram matrix C = g^T . x, summed over the tokens.
// Also dL/dcs_j = (R . C)[j][j] and dL/dx = g . R'^T with R' = diag(cs) . R.
//
// So every token enters only two contractions on the matrix cores, C = g^T x
// (bwd_gram_kernel) and g . R'^T (bwd_dx_kernel), and the stage walk runs on
// the 128 rows of C per group instead of on every token (bwd_walk_kernel).
// The walk is row-parallel: with u_i = column i of C,
//   (R . C)[:, i]   = R u_i          (stages applied to u_i as a column,
//                                     last stage first: inverse rotations)
//   row i of N_0^T  = v_i = cs_i (R u_i)
//   row i of F_t    = f_i = e_i . R_1 ... R_t      (forward rotations)
//   dL/dtheta_t(p)  = sum over i of f_i[b] (v_i R_1..R_t)[a] - f_i[a] (v_i R_1..R_t)[b]
// (from N_t^T = F_t^T N_0^T F_t), and after the last stage f_i is row i of R,
// which gives R' for the dL/dx product.  Sums over tokens and over rows are
// taken in a fixed order, so results are identical from call to call.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace paro {

constexpr int kBwdTok = 64;                  // token granule of the Gram splits
// tokens per LDS tile of the Gram kernel (128-token tiles measured slower:
// fewer splits in flight, the same transposing LDS writes per token)
__host__ __device__ constexpr int gram_tile(int) { return kBwdTok; }
constexpr int kWalkRows = 8;                 // rows of C per wave in the walk
constexpr int kWalkParts = kG / kWalkRows;   // dtheta partial rows per group
constexpr int kBwdRS = kG + 4;               // walk LDS row stride (floats)
constexpr int kDxHS = kG + 8;                // dx LDS row stride of H / L (halves)
constexpr int kDxRows = 512;                 // tokens per dx workgroup
constexpr int64_t kBwdMat = 2 * kG * kG;     // H and L of one group (halves)
constexpr int kGramTarget = 512;             // Gram workgroups to aim for

// Matrix-core dtype of each product: fp16 when both operands are fp16
// (exact), otherwise bf16 with fp16 / fp32 operands split into a bf16 high
// part and a bf16 remainder (fp16: exact in two parts; fp32: to 2^-17).
__host__ __device__ constexpr int gram_mdt(int xdt, int gdt) { return (xdt == kF16 && gdt == kF16) ? kF16 : kBF16; }
__host__ __device__ constexpr int dx_mdt(int gdt) { return gdt == kF16 ? kF16 : kBF16; }

__device__ __forceinline__ int mfma_row_of_channel(int j) {
  // inverse of the dx output order: MFMA row 32b + 16h + 4q + r holds channel 32b + 8q + 4h + r
  return (j & ~31) | (((j >> 2) & 1) << 4) | (((j >> 3) & 3) << 2) | (j & 3);
}

// ---------------------------------------------------------------------------
// Gram kernel: C^T[i][k] = sum over tokens of x[m][i] * g[m][k], one 128 x 128
// fp32 partial per (group, token split).  Tiles of 64 tokens are loaded with
// coalesced 16-byte reads and written to LDS transposed (channel-major, eight
// tokens per 16-byte block, blocks XOR-swizzled by the channel's 8-block), so
// that each MFMA fragment (one channel, eight consecutive tokens) is one
// 16-byte LDS read.  Wave w owns C^T rows 32w..32w+31 (two 16-row tiles) and
// all 128 columns: 16 accumulator tiles.
// ---------------------------------------------------------------------------
template <int T>
__device__ __forceinline__ int gram_off(int ch, int tok) {
  return ch * T + ((((tok >> 3) ^ (ch >> 3)) & (T / 8 - 1)) << 3) + (tok & 7);
}

template <int XDT, int GDT>
__global__ void __launch_bounds__(256, 2)
bwd_gram_kernel(const void *__restrict__ x, const void *__restrict__ gin, int64_t tokens, int64_t I,
                int64_t chunk, float *__restrict__ cpart) {
  constexpr int MD = gram_mdt(XDT, GDT);
  constexpr int XP = (XDT == kF16 && MD == kBF16) ? 2 : 1;  // parts of x
  constexpr int GP = (GDT == kF32 || (GDT == kF16 && MD == kBF16)) ? 2 : 1;
  constexpr int T = gram_tile(GDT);
  constexpr int XCH = T / 16;                          // 16-byte chunks of x per thread and tile
  constexpr int GCH = GDT == kF32 ? T / 8 : T / 16;    // and of g
  __shared__ __attribute__((aligned(16))) uint16_t xt[XP][kG * T];
  __shared__ __attribute__((aligned(16))) uint16_t gt[GP][kG * T];

  const int tid = threadIdx.x, lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t g = blockIdx.x, groups = I / kG;
  const int64_t m_begin = (int64_t)blockIdx.y * chunk;
  const int64_t m_end = tokens < m_begin + chunk ? tokens : m_begin + chunk;
  const int gsz = GDT == kF32 ? 4 : 2;

  u32x4 xr[XCH], gr[GCH];
  auto load_tile = [&](int64_t m0) {
    const int64_t rows = m_end - m0 < T ? m_end - m0 : T;  // > 0
    const __amdgpu_buffer_rsrc_t rx =
        raw_rsrc(reinterpret_cast<const uint16_t *>(x) + m0 * I + g * kG, (uint32_t)(rows * I * 2));
    const __amdgpu_buffer_rsrc_t rg =
        raw_rsrc(reinterpret_cast<const char *>(gin) + (m0 * I + g * kG) * gsz, (uint32_t)(rows * I * gsz));
#pragma unroll
    for (int u = 0; u < XCH; ++u) {
      const int c = tid + 256 * u, row = c >> 4, cb = c & 15;
      xr[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)((row * I + cb * 8) * 2), 0, 0);
    }
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
      const int c = tid + 256 * u;
      const int row = GDT == kF32 ? c >> 5 : c >> 4, cb = GDT == kF32 ? c & 31 : c & 15;
      gr[u] = __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)((row * I) * gsz + cb * 16), 0, 0);
    }
  };

  auto put = [&](uint16_t *arr, int ch, int tok, uint32_t v) { arr[gram_off<T>(ch, tok)] = (uint16_t)v; };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < XCH; ++u) {
      const int c = tid + 256 * u, tok = c >> 4, cb = c & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = (xr[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        if constexpr (XP == 1) {
          put(xt[0], 8 * cb + e, tok, h);
        } else {  // fp16 -> bf16 high part + exact bf16 remainder
          const float v = f16_bits_to_f32(h);
          const uint32_t hi = f32_to_bf16_bits(v);
          put(xt[0], 8 * cb + e, tok, hi);
          put(xt[XP - 1], 8 * cb + e, tok, f32_to_bf16_bits(v - bf16_bits_to_f32(hi)));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
      const int c = tid + 256 * u;
      if constexpr (GDT == kF32) {
        const int tok = c >> 5, cb = c & 31;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = __uint_as_float(gr[u][e]);
          const uint32_t hi = f32_to_bf16_bits(v);
          put(gt[0], 4 * cb + e, tok, hi);
          put(gt[GP - 1], 4 * cb + e, tok, f32_to_bf16_bits(v - bf16_bits_to_f32(hi)));
        }
      } else {
        const int tok = c >> 4, cb = c & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t h = (gr[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          if constexpr (GP == 1) {
            put(gt[0], 8 * cb + e, tok, h);
          } else {
            const float v = f16_bits_to_f32(h);
            const uint32_t hi = f32_to_bf16_bits(v);
            put(gt[0], 8 * cb + e, tok, hi);
            put(gt[GP - 1], 8 * cb + e, tok, f32_to_bf16_bits(v - bf16_bits_to_f32(hi)));
          }
        }
      }
    }
  };

  f32x4 acc[2][8];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      acc[it][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_fence(acc[it][kt]);
    }
  asm volatile("s_nop 7");

  const int fr = lane & 15, fj = lane >> 4;
  auto frag = [&](const uint16_t *arr, int ch, int j) {
    return *reinterpret_cast<const u32x4 *>(arr + ch * T + (((j ^ (ch >> 3)) & (T / 8 - 1)) << 3));
  };

  if (m_begin < m_end) load_tile(m_begin);
  for (int64_t m0 = m_begin; m0 < m_end; m0 += T) {
    __syncthreads();  // the previous tile's fragments are read
    asm volatile("s_nop 7");  // before VALU reuses registers the last asm MFMAs read
    __builtin_amdgcn_sched_barrier(0);
    store_tile();
    if (m0 + T < m_end) load_tile(m0 + T);  // in flight during the products below
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < T / 32; ++ks) {
      const int j = 4 * ks + fj;
      u32x4 a[2][XP];
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int p = 0; p < XP; ++p) a[it][p] = frag(xt[p], 32 * wave + 16 * it + fr, j);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        u32x4 b[GP];
#pragma unroll
        for (int p = 0; p < GP; ++p) b[p] = frag(gt[p], 16 * kt + fr, j);
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int xp = 0; xp < XP; ++xp)
#pragma unroll
            for (int gp = 0; gp < GP; ++gp) mfma_acc<MD>(a[it][xp], b[gp], acc[it][kt]);
      }
    }
  }
  mfma_drain();
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) acc_fence(acc[it][kt]);

  // lane l of tile (it, kt): rows 32w + 16it + 4(l/16) + r, column 16kt + l%16
  float *out = cpart + ((int64_t)blockIdx.y * groups + g) * (kG * kG);
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(32 * wave + 16 * it + 4 * fj + r) * kG + 16 * kt + fr] = acc[it][kt][r];
}

// ---------------------------------------------------------------------------
// Walk kernel: rows i of C^T (columns of C) of one group, 8 per wave, four
// workgroups per group.  Lane p owns pair p of every stage (as in the forward
// rotation).  Writes dL/dcs_i, the wave's dtheta partial sums and row i of
// R' = diag(cs) R as H + L (dtype MDT) at its MFMA row for the dx product.
// ---------------------------------------------------------------------------
template <int MDT>
__global__ void __launch_bounds__(256)
bwd_walk_kernel(const float *__restrict__ cpart, int splits, int64_t I, const int16_t *__restrict__ pairs,
                const float *__restrict__ theta, const float *__restrict__ cscale, int krot, int gmask,
                float *__restrict__ gcs, float *__restrict__ tpart, uint16_t *__restrict__ hl) {
  constexpr int RW = kWalkRows;
  __shared__ float lds[4][2][RW * kBwdRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x, groups = I / kG;
  const int i0 = blockIdx.y * (4 * RW) + wave * RW;
  float *vs = lds[wave][0], *fs = lds[wave][1];
  const int16_t *pairs_g = pairs + g * kG;
  const float *theta_g = theta + g * kPairs;

  // parameters of the last kStageRegs stages (the inverse walk starts there)
  uint32_t pw[kStageRegs];
  float th[kStageRegs];
#pragma unroll
  for (int u = 0; u < kStageRegs; ++u) {
    const int t = krot - 1 - u >= 0 ? krot - 1 - u : 0;
    pw[u] = load_pair_word(pairs_g, I, t, lane, gmask);
    th[u] = theta_g[(int64_t)t * (I / 2) + lane];
  }

  // u_i = column i of C = row i of C^T, the token splits added in order;
  // four splits' loads of all rows are in flight at a time
  float2 us[RW];
#pragma unroll
  for (int m = 0; m < RW; ++m) us[m] = float2{0.f, 0.f};
  const float *crow = cpart + (g * kG + i0) * kG + 2 * lane;
  const int64_t split_stride = groups * kG * kG;
  for (int sp0 = 0; sp0 < splits; sp0 += 4) {
    float2 v[4][RW];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int m = 0; m < RW; ++m)
        v[q][m] = sp0 + q < splits ? *reinterpret_cast<const float2 *>(crow + (sp0 + q) * split_stride + m * kG)
                                   : float2{0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int m = 0; m < RW; ++m) {
        us[m].x += v[q][m].x;
        us[m].y += v[q][m].y;
      }
  }
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    vs[m * kBwdRS + 2 * lane] = us[m].x;
    vs[m * kBwdRS + 2 * lane + 1] = us[m].y;
  }
  wave_lds_sync();

  // R u_i: each stage applied to the column, last stage first (inverse rotations)
#pragma unroll
  for (int u = 0; u < kStageRegs; ++u) {
    if (u < krot) {
      float c, sn;
      __sincosf(th[u], &sn, &c);
      rotate_stage<RW>(vs, kBwdRS, pw[u], c, -sn);
    }
  }
  for (int t = krot - 1 - kStageRegs; t >= 0; --t) {
    const uint32_t w = load_pair_word(pairs_g, I, t, lane, gmask);
    float c, sn;
    __sincosf(theta_g[(int64_t)t * (I / 2) + lane], &sn, &c);
    rotate_stage<RW>(vs, kBwdRS, w, c, -sn);
  }

  // dL/dcs_i = (R C)[i][i]; then v_i = cs_i (R u_i) and f_i = e_i
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const int i = i0 + m;
    if ((i >> 1) == lane) gcs[g * kG + i] = vs[m * kBwdRS + i];
  }
  float csr[RW];
#pragma unroll
  for (int m = 0; m < RW; ++m) csr[m] = cscale[g * kG + i0 + m];
  wave_lds_sync();
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    vs[m * kBwdRS + 2 * lane] *= csr[m];
    vs[m * kBwdRS + 2 * lane + 1] *= csr[m];
    fs[m * kBwdRS + 2 * lane] = 2 * lane == i0 + m ? 1.0f : 0.0f;
    fs[m * kBwdRS + 2 * lane + 1] = 2 * lane + 1 == i0 + m ? 1.0f : 0.0f;
  }
  wave_lds_sync();

  // forward stages on v_i and f_i; after stage t, lane p adds
  // f_i[b] v_i[a] - f_i[a] v_i[b] over the wave's rows
  RotParams rp;
  rp.load(pairs_g, I, theta_g, I / 2, krot, lane, gmask);
  float *prow = tpart + ((int64_t)blockIdx.y * 4 + wave) * ((int64_t)krot * (I / 2)) + g * kPairs + lane;
  for (int t = 0; t < krot; ++t) {
    uint32_t w;
    float tht;
    if (t < kStageRegs) {
      w = rp.pw[0];
      tht = rp.th[0];
#pragma unroll
      for (int u = 1; u < kStageRegs; ++u)
        if (t == u) {
          w = rp.pw[u];
          tht = rp.th[u];
        }
    } else {
      w = load_pair_word(pairs_g, I, t, lane, gmask);
      tht = theta_g[(int64_t)t * (I / 2) + lane];
    }
    float c, s;
    __sincosf(tht, &s, &c);
    const int a = (int)(w & (kG - 1)), b = (int)((w >> 16) & (kG - 1));
    float va[RW], vb[RW], fa[RW], fb[RW];
#pragma unroll
    for (int m = 0; m < RW; ++m) {
      va[m] = vs[m * kBwdRS + a];
      vb[m] = vs[m * kBwdRS + b];
      fa[m] = fs[m * kBwdRS + a];
      fb[m] = fs[m * kBwdRS + b];
    }
    float dth = 0.0f;
#pragma unroll
    for (int m = 0; m < RW; ++m) {
      const float va2 = __builtin_fmaf(va[m], c, vb[m] * s), vb2 = __builtin_fmaf(vb[m], c, -(va[m] * s));
      const float fa2 = __builtin_fmaf(fa[m], c, fb[m] * s), fb2 = __builtin_fmaf(fb[m], c, -(fa[m] * s));
      dth = __builtin_fmaf(fb2, va2, __builtin_fmaf(-fa2, vb2, dth));
      vs[m * kBwdRS + a] = va2;
      vs[m * kBwdRS + b] = vb2;
      fs[m * kBwdRS + a] = fa2;
      fs[m * kBwdRS + b] = fb2;
    }
    prow[(int64_t)t * (I / 2)] = dth;
    wave_lds_sync();
  }

  // f_i is now row i of R: R'[i][:] = cs_i f_i as H + L at MFMA row r(i)
  uint32_t *hg = reinterpret_cast<uint32_t *>(hl + g * kBwdMat) + lane;
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const int r = mfma_row_of_channel(i0 + m);
    const float v0 = fs[m * kBwdRS + 2 * lane] * csr[m], v1 = fs[m * kBwdRS + 2 * lane + 1] * csr[m];
    const uint32_t hb = pack2<MDT>(v0, v1);
    const float e0 = v0 - act_to_f32<MDT>(hb & 0xffffu), e1 = v1 - act_to_f32<MDT>(hb >> 16);  // exact
    hg[r * (kG / 2)] = hb;
    hg[(kG + r) * (kG / 2)] = pack2<MDT>(e0, e1);
  }
}

// ---------------------------------------------------------------------------
// dx kernel: dL/dx = g . R'^T per group on the matrix cores, computed as its
// transpose R' . g^T with H / L (rows of R' in MFMA order) as the A operand
// and g's rows as B fragments.  Lane l of row tile t then holds, for its token
// l%16, the 8 consecutive channels 32b + 8(l/16) .. +7 of each 32-channel
// block b: one 16-byte (32-byte for fp32) row-major store each.  fp32 g is
// split into a bf16 high part and remainder: H.hi + H.lo + L.hi.
// ---------------------------------------------------------------------------
template <int GDT, int ODT>
__global__ void __launch_bounds__(256, 2)
bwd_dx_kernel(const void *__restrict__ gin, void *__restrict__ gx, int64_t tokens, int64_t I,
              const uint16_t *__restrict__ hl) {
  constexpr int MD = dx_mdt(GDT);
  constexpr bool F32G = GDT == kF32;
  constexpr int TB = F32G ? 2 : 4;  // row tiles per wave and batch
  constexpr int gsz = F32G ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t hlds[2 * kG * kDxHS];
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t g = blockIdx.x;
  const int64_t mt_end = (tokens + 15) / 16;
  const int64_t mt_first = (int64_t)blockIdx.y * (kDxRows / 16);
  const int64_t mt_last = mt_first + kDxRows / 16 < mt_end ? mt_first + kDxRows / 16 : mt_end;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const uint32_t lane_off = (uint32_t)((fr * I + fk) * gsz);

  // raw g fragments: [tile][k-step][1 or 2 x 16 bytes]
  constexpr int NPC = F32G ? 2 : 1;
  u32x4 raw[TB][4][NPC];
  auto load_g = [&](int64_t mt0, int ks, bool all) {
    const int64_t row0 = mt0 * 16;
    const int64_t rows = tokens - row0 < 16 * TB ? tokens - row0 : 16 * TB;
    const __amdgpu_buffer_rsrc_t r =
        raw_rsrc(reinterpret_cast<const char *>(gin) + (row0 * I + g * kG) * gsz, (uint32_t)(rows * I * gsz));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!all && k != ks) continue;
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int h = 0; h < NPC; ++h)
          raw[t][k][h] = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, (int)((t * 16 * I + k * 32) * gsz + 16 * h), 0);
    }
  };

  int64_t mt0 = mt_first + wave * TB;
  if (mt0 < mt_last) load_g(mt0, 0, true);

  const uint16_t *hg = hl + g * kBwdMat;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = threadIdx.x + 256 * (8 * half + u);  // matrix row c/16 (of 256), 16-byte part c%16
      const u32x4 v = *reinterpret_cast<const u32x4 *>(hg + (int64_t)c * 8);
      *reinterpret_cast<u32x4 *>(hlds + (c >> 4) * kDxHS + (c & 15) * 8) = v;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  constexpr int kStride = 4 * TB;
  for (; mt0 < mt_last; mt0 += kStride) {
    const int64_t next = mt0 + kStride;
    const bool more = next < mt_last;
    f32x4 acc[TB][8];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        acc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_fence(acc[t][ct]);
      }
    asm volatile("s_nop 7");
    auto read_a = [&](int step) {
      const int ks = step >> 4, ct = (step >> 1) & 7, hlm = step & 1;
      return *reinterpret_cast<const u32x4 *>(hlds + (hlm * kG + ct * 16 + fr) * kDxHS + ks * 32 + fk);
    };
    u32x4 ar[3];
    ar[0] = read_a(0);
    ar[1] = read_a(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // this k-step's B fragments (fp32 g: bf16 high part and remainder)
      u32x4 hi[TB], lo[TB];
      if constexpr (F32G) {
        // the conversion writes registers that the previous k-step's MFMAs
        // read; the compiler does not see those asm MFMAs
        if (ks > 0) asm volatile("s_nop 7");
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if constexpr (F32G) {
          uint32_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x4 &src = raw[t][ks][e >> 1];
            const float v0 = __uint_as_float(src[2 * (e & 1)]), v1 = __uint_as_float(src[2 * (e & 1) + 1]);
            h[e] = pack2<kBF16>(v0, v1);
            l[e] = pack2<kBF16>(v0 - bf16_bits_to_f32(h[e] & 0xffffu), v1 - bf16_bits_to_f32(h[e] >> 16));
          }
          hi[t] = u32x4{h[0], h[1], h[2], h[3]};
          lo[t] = u32x4{l[0], l[1], l[2], l[3]};
        } else {
          hi[t] = raw[t][ks][0];
        }
      }
#pragma unroll
      for (int sub = 0; sub < 16; ++sub) {
        const int step = ks * 16 + sub, ct = sub >> 1, hlm = sub & 1;
        if (step + 2 < 64) ar[(step + 2) % 3] = read_a(step + 2);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          mfma_acc<MD>(ar[step % 3], hi[t], acc[t][ct]);
          if constexpr (F32G) {
            if (hlm == 0) mfma_acc<MD>(ar[step % 3], lo[t], acc[t][ct]);
          }
        }
        if (sub == 15 && more) load_g(next, ks, false);  // k-step consumed: next batch's fragments
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_drain();
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc_fence(acc[t][ct]);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int64_t tok = (mt0 + t) * 16 + fr;
      if (tok < tokens) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x4 l4 = acc[t][2 * b], h4 = acc[t][2 * b + 1];
          const int64_t off = tok * I + g * kG + 32 * b + fk;
          if constexpr (ODT == kF32) {
            float *o = reinterpret_cast<float *>(gx) + off;
            __builtin_nontemporal_store(l4, reinterpret_cast<f32x4 *>(o));
            __builtin_nontemporal_store(h4, reinterpret_cast<f32x4 *>(o + 4));
          } else {
            const u32x4 v{pack2<ODT>(l4[0], l4[1]), pack2<ODT>(l4[2], l4[3]), pack2<ODT>(h4[0], h4[1]),
                          pack2<ODT>(h4[2], h4[3])};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(gx) + off));
          }
        }
      }
    }
  }
}

// gtheta[e] = sum over the kWalkParts partial rows, in order
__global__ void __launch_bounds__(256)
bwd_theta_reduce_kernel(const float *__restrict__ tpart, int64_t n, float *__restrict__ gtheta) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.0f;
#pragma unroll
  for (int p = 0; p < kWalkParts; ++p) s += tpart[p * n + e];
  gtheta[e] = s;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
int64_t gram_splits(int64_t tokens, int64_t I) {
  const int64_t groups = I / kG, tiles = (tokens + kBwdTok - 1) / kBwdTok;
  int64_t s = (kGramTarget + groups - 1) / groups;
  if (s > tiles) s = tiles;
  return s < 1 ? 1 : s;
}
size_t align256(size_t v) { return (v + 255) / 256 * 256; }
struct BwdLayout {
  int64_t splits, chunk;
  size_t hl_off, c_off, t_off, total;
};
BwdLayout bwd_layout(int64_t tokens, int64_t I, int krot) {
  BwdLayout L;
  L.splits = gram_splits(tokens, I);
  const int64_t tiles = (tokens + kBwdTok - 1) / kBwdTok;
  L.chunk = ((tiles + L.splits - 1) / L.splits) * kBwdTok;
  if (L.chunk == 0) L.chunk = kBwdTok;
  L.hl_off = 0;
  L.c_off = align256((size_t)(I / kG) * kBwdMat * 2);
  L.t_off = L.c_off + align256((size_t)L.splits * (size_t)(I / kG) * kG * kG * 4);
  L.total = L.t_off + align256((size_t)kWalkParts * (size_t)krot * (size_t)(I / 2) * 4);
  return L;
}
}  // namespace

size_t rot_backward_partial_bytes(int64_t tokens, int64_t I, int krot) { return bwd_layout(tokens, I, krot).total; }

template <int XDT, int GDT>
static void launch_gram(dim3 grid, hipStream_t st, const void *x, const void *g, int64_t tokens, int64_t I,
                        int64_t chunk, float *cpart) {
  hipLaunchKernelGGL((bwd_gram_kernel<XDT, GDT>), grid, dim3(256), 0, st, x, g, tokens, I, chunk, cpart);
}

template <int GDT>
static void launch_dx(int gx_dt, dim3 grid, hipStream_t st, const void *g, void *gx, int64_t tokens, int64_t I,
                      const uint16_t *hl) {
  if (gx_dt == kF32)
    hipLaunchKernelGGL((bwd_dx_kernel<GDT, kF32>), grid, dim3(256), 0, st, g, gx, tokens, I, hl);
  else if (gx_dt == kF16)
    hipLaunchKernelGGL((bwd_dx_kernel<GDT, kF16>), grid, dim3(256), 0, st, g, gx, tokens, I, hl);
  else
    hipLaunchKernelGGL((bwd_dx_kernel<GDT, kBF16>), grid, dim3(256), 0, st, g, gx, tokens, I, hl);
}

hipError_t launch_rot_backward(const void *x, int x_dt, const void *gin, int g_dt, int64_t tokens, int64_t I,
                               const int16_t *pairs, const float *theta, const float *cs, int krot, int group,
                               void *gx, int gx_dt, float *gtheta, float *gcs, float *partial, hipStream_t st) {
  const BwdLayout L = bwd_layout(tokens, I, krot);
  char *ws = reinterpret_cast<char *>(partial);
  uint16_t *hl = reinterpret_cast<uint16_t *>(ws + L.hl_off);
  float *cpart = reinterpret_cast<float *>(ws + L.c_off);
  float *tpart = reinterpret_cast<float *>(ws + L.t_off);
  const unsigned groups = (unsigned)(I / kG);

  // 1. Gram partials (with no tokens: one split of zeros)
  const dim3 ggrid(groups, (unsigned)L.splits);
  if (x_dt == kF16) {
    if (g_dt == kF32) launch_gram<kF16, kF32>(ggrid, st, x, gin, tokens, I, L.chunk, cpart);
    else launch_gram<kF16, kF16>(ggrid, st, x, gin, tokens, I, L.chunk, cpart);
  } else {
    if (g_dt == kF32) launch_gram<kBF16, kF32>(ggrid, st, x, gin, tokens, I, L.chunk, cpart);
    else launch_gram<kBF16, kBF16>(ggrid, st, x, gin, tokens, I, L.chunk, cpart);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 2. the stage walk: dL/dcs, dtheta partials, R' for the dx product
  const dim3 wgrid(groups, kG / (4 * kWalkRows));
  if (dx_mdt(g_dt) == kF16)
    hipLaunchKernelGGL((bwd_walk_kernel<kF16>), wgrid, dim3(256), 0, st, cpart, (int)L.splits, I, pairs, theta, cs,
                       krot, kG - group, gcs, tpart, hl);
  else
    hipLaunchKernelGGL((bwd_walk_kernel<kBF16>), wgrid, dim3(256), 0, st, cpart, (int)L.splits, I, pairs, theta,
                       cs, krot, kG - group, gcs, tpart, hl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 3. dL/dx
  if (tokens > 0) {
    const dim3 dgrid(groups, (unsigned)((tokens + kDxRows - 1) / kDxRows));
    if (g_dt == kF32) launch_dx<kF32>(gx_dt, dgrid, st, gin, gx, tokens, I, hl);
    else if (g_dt == kF16) launch_dx<kF16>(gx_dt, dgrid, st, gin, gx, tokens, I, hl);
    else launch_dx<kBF16>(gx_dt, dgrid, st, gin, gx, tokens, I, hl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // 4. dL/dtheta
  const int64_t n = (int64_t)krot * (I / 2);
  hipLaunchKernelGGL(bwd_theta_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tpart, n, gtheta);
  return hipGetLastError();
}

}  // namespace paro

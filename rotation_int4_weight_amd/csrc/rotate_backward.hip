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
// and g . R'^T, both taken in one pass over the tokens (bwd_gram_dx_kernel:
// x and g are read once, dL/dx written once), and the stage walk runs on the
// 128 rows of C per group instead of on every token (bwd_walk_kernel).  R'
// depends only on the angles and scales, so it is formed first
// (bwd_rrow_kernel: row i of R is e_i pushed forward through the stages).
// The walk is row-parallel: with u_i = column i of C,
//   (R . C)[:, i]   = R u_i          (stages applied to u_i as a column,
//                                     last stage first: inverse rotations)
//   row i of N_0^T  = v_i = cs_i (R u_i)
//   row i of F_t    = f_i = e_i . R_1 ... R_t      (forward rotations)
//   dL/dtheta_t(p)  = sum over i of f_i[b] (v_i R_1..R_t)[a] - f_i[a] (v_i R_1..R_t)[b]
// (from N_t^T = F_t^T N_0^T F_t).  Sums over tokens and over rows are taken
// in a fixed order, so results are identical from call to call.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace paro {

constexpr int kFT = 64;                      // tokens per tile of the fused kernel (the split granule)
constexpr int kWalkRows = 8;                 // rows of C per wave in the walk
constexpr int kWalkParts = kG / kWalkRows;   // dtheta partial rows per group
constexpr int kBwdRS = kG + 4;               // walk / build LDS row stride (floats)
constexpr int kRowsPerBuild = 16;            // rows of R' per one-wave build workgroup
constexpr int64_t kBwdMat = 2 * kG * kG;     // H and L of one group (halves)
constexpr int kGramResident = 256;           // fused workgroups that fit the chip at once

// Matrix-core dtype of each product: fp16 when both operands are fp16
// (exact), otherwise bf16 with fp16 / fp32 operands split into a bf16 high
// part and a bf16 remainder (fp16: exact in two parts; fp32: to 2^-17).
__host__ __device__ constexpr int gram_mdt(int xdt, int gdt) { return (xdt == kF16 && gdt == kF16) ? kF16 : kBF16; }
__host__ __device__ constexpr int dx_mdt(int gdt) { return gdt == kF16 ? kF16 : kBF16; }

// MFMA row 32b + 16h + 4q + r (b < 4, h < 2, q < 4, r < 4) of R' holds
// channel 32b + 8q + 4h + r: the dL/dx accumulators of row tiles 2b and 2b+1
// then give each lane 8 consecutive channels of one token.
__device__ __forceinline__ int channel_of_row(int r) {
  return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

// ---------------------------------------------------------------------------
// R' build: one wave forms rows r0 = 16 * blockIdx.y .. r0+15 (MFMA order) of
// R' = diag(cs) . R for group blockIdx.x.  Row i of R is the unit row e_i
// through the forward stages (the same staged fp32 code as the forward
// rotation); times cs_i it is stored as H + L in dtype MDT, H = rne(R'),
// L = rne(R' - H).
// hl: [group][2 (H, L)][128 (MFMA row)][128 (channel j)], R'[i][j].
// ---------------------------------------------------------------------------
template <int MDT>
__global__ void __launch_bounds__(64)
bwd_rrow_kernel(int64_t I, const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                const float *__restrict__ cscale, int krot, int gmask, uint16_t *__restrict__ hl) {
  constexpr int RW = kRowsPerBuild;
  __shared__ float xs[RW * kBwdRS];
  const int lane = lane_id();
  const int64_t g = blockIdx.x;
  const int r0 = blockIdx.y * RW;
  const int16_t *pairs_g = pairs + g * kG;
  const float *theta_g = theta + g * kPairs;
  RotParams rp;
  rp.load(pairs_g, I, theta_g, I / 2, krot, lane, gmask);
  float csr[RW];
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const int i = channel_of_row(r0 + m);
    csr[m] = cscale[g * kG + i];
    xs[m * kBwdRS + 2 * lane] = 2 * lane == i ? 1.0f : 0.0f;
    xs[m * kBwdRS + 2 * lane + 1] = 2 * lane + 1 == i ? 1.0f : 0.0f;
  }
  wave_lds_sync();
  rotate_rows_lds<RW>(xs, kBwdRS, rp, pairs_g, I, theta_g, I / 2, krot, lane, gmask);
  uint32_t *hg = reinterpret_cast<uint32_t *>(hl + g * kBwdMat) + lane;
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const float v0 = xs[m * kBwdRS + 2 * lane] * csr[m], v1 = xs[m * kBwdRS + 2 * lane + 1] * csr[m];
    const uint32_t hb = pack2<MDT>(v0, v1);
    const float e0 = v0 - act_to_f32<MDT>(hb & 0xffffu), e1 = v1 - act_to_f32<MDT>(hb >> 16);  // exact
    hg[(r0 + m) * (kG / 2)] = hb;
    hg[(kG + r0 + m) * (kG / 2)] = pack2<MDT>(e0, e1);
  }
}

// ---------------------------------------------------------------------------
// Fused Gram + dL/dx kernel: one workgroup of 8 waves per (group, token
// split); tiles of 64 tokens of x and g are read once (coalesced 16-byte
// loads), two tiles ahead of the products (two register sets, the tile loop
// unrolled by two so that each set keeps its registers; one tile ahead for
// fp32 g, whose fragments take twice the registers).
//
//  * Loads: wave w takes tokens 32s .. 32s+31 (s = w / 4) and channels
//    32c .. 32c+31 (c = w % 4) of the tile, as MFMA A fragments in natural
//    order (lane l: token l%16 of a 16-token block, 8 consecutive channels).
//  * Transpose on the matrix cores: an MFMA of such a fragment with a one-hot
//    B (B[k][n] = 1 where k = 16h + n) returns, exactly in fp32, lane l's
//    channel 16h + l%16 at tokens 4(l/16) .. +3 of the block.  Two blocks'
//    results packed together are one 16-byte, channel-major LDS store: eight
//    tokens of one channel, the k-slots of a Gram fragment.  x and g go
//    through the same token-to-slot map, so their products pair up right.
//    (A non-finite input value spreads through the zeros of the one-hot
//    operand to its 16-channel block of that token.)
//  * Gram: wave w owns the 32 x 64 block of C^T at rows 32(w/2) (x channels)
//    and columns 64(w%2) (g channels): 8 accumulator tiles over the split.
//  * dL/dx = g . R'^T as its transpose R' . g^T: wave w holds rows 32(w%4) ..
//    +31 of R' (H and L, MFMA order) in registers as A fragments and takes
//    tokens 32(w/4) .. +31; g in natural order from LDS gives the B
//    fragments.  Lane l's accumulators are then 8 consecutive channels of one
//    token: a 16-byte (fp32: 32-byte) store.
//  LDS slots are XOR-swizzled so that every 16-lane quarter of a 16-byte LDS
//  access covers all 64 banks.  Under register pressure (fp32 g) the
//  allocator keeps some R' fragments in AGPRs and copies them out right
//  before use, so every product here waits out a VALU write first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_to_bf16(const float *v, u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = pack2<kBF16>(v[2 * e], v[2 * e + 1]);
    hi[e] = h;
    lo[e] = pack2<kBF16>(v[2 * e] - bf16_bits_to_f32(h & 0xffffu), v[2 * e + 1] - bf16_bits_to_f32(h >> 16));
  }
}

template <int N>
struct Const {
  static constexpr int value = N;
};

template <int XDT, int GDT>
__global__ void __launch_bounds__(512)
bwd_gram_dx_kernel(const void *__restrict__ x, const void *__restrict__ gin, void *__restrict__ gx, int gx_f32,
                   int64_t tokens, int64_t I, int64_t chunk, const uint16_t *__restrict__ hl,
                   float *__restrict__ cpart) {
  constexpr int MG = gram_mdt(XDT, GDT), MX = dx_mdt(GDT);
  constexpr bool F32G = GDT == kF32;
  constexpr int XP = XDT == MG ? 1 : 2;  // parts of x in MG
  constexpr int GP = F32G ? 2 : 1;       // parts of g (in MG = MX for fp32 g)
  constexpr int gsz = F32G ? 4 : 2;
  constexpr int PF = F32G ? 1 : 2;  // tiles in flight ahead of the products (register sets)
  __shared__ __attribute__((aligned(16))) uint16_t xt[XP][kG * kFT];  // [channel][8 slots of 8 tokens]
  __shared__ __attribute__((aligned(16))) uint16_t gt[GP][kG * kFT];
  __shared__ __attribute__((aligned(16))) uint16_t gn[GP][kFT * kG];  // [token][16 slots of 8 channels]

  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int fr = lane & 15, q = lane >> 4;
  const int64_t g = blockIdx.x, groups = I / kG;
  const int64_t m_begin = (int64_t)blockIdx.y * chunk;
  const int64_t m_end = tokens < m_begin + chunk ? tokens : m_begin + chunk;
  const int ls = wave >> 2, lc = wave & 3;   // load role
  const int gi = wave >> 1, gk = wave & 1;   // Gram role
  const int dr = wave & 3, dt = wave >> 2;   // dL/dx role

  // rows 32 dr + 16it + fr of R' (H, L): A fragments of the dL/dx product
  u32x4 ar[2][4][2];
  {
    const uint16_t *hg = hl + g * kBwdMat;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          ar[it][ks][p] =
              *reinterpret_cast<const u32x4 *>(hg + ((int64_t)p * kG + 32 * dr + 16 * it + fr) * kG + 32 * ks + 8 * q);
  }
  // one-hot B fragments: element e of lane l is 1 where 8(l/16) + e = 16h + l%16
  constexpr uint32_t kOne = MG == kF16 ? 0x3c00u : 0x3f80u;
  u32x4 oh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 16 * h + fr - 8 * q;
#pragma unroll
    for (int k = 0; k < 4; ++k) oh[h][k] = (e >> 1) == k ? kOne << (16 * (e & 1)) : 0u;
  }

  u32x4 xr[PF][2], gr[PF][2][GP];  // [register set][16-token block][...]
  auto load_tile = [&](auto set, int64_t m0) {
    constexpr int S = decltype(set)::value;
    const int64_t rows = m_end - m0 < kFT ? m_end - m0 : kFT;  // > 0; later rows read as zeros
    const __amdgpu_buffer_rsrc_t rx =
        raw_rsrc(reinterpret_cast<const uint16_t *>(x) + m0 * I + g * kG, (uint32_t)(rows * I * 2));
    const __amdgpu_buffer_rsrc_t rg =
        raw_rsrc(reinterpret_cast<const char *>(gin) + (m0 * I + g * kG) * gsz, (uint32_t)(rows * I * gsz));
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t e = (uint32_t)((32 * ls + 16 * tt + fr) * I + 32 * lc + 8 * q);
      xr[S][tt] = __builtin_amdgcn_raw_buffer_load_b128(rx, e * 2, 0, 0);
#pragma unroll
      for (int h = 0; h < GP; ++h) gr[S][tt][h] = __builtin_amdgcn_raw_buffer_load_b128(rg, e * gsz + 16 * h, 0, 0);
    }
  };

  // parts, the natural copy of g, the transposes
  auto store_tile = [&](auto set) {
    constexpr int S = decltype(set)::value;
    u32x4 xp[2][XP], gp[2][GP];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if constexpr (XP == 1) {
        xp[tt][0] = xr[S][tt];
      } else {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f16_bits_to_f32((xr[S][tt][e >> 1] >> (16 * (e & 1))) & 0xffffu);
        split_to_bf16(v, xp[tt][0], xp[tt][1]);
      }
      if constexpr (F32G) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(gr[S][tt][e >> 2][e & 3]);
        split_to_bf16(v, gp[tt][0], gp[tt][1]);
      } else {
        gp[tt][0] = gr[S][tt][0];
      }
      const int tok = 32 * ls + 16 * tt + fr;
#pragma unroll
      for (int p = 0; p < GP; ++p)
        *reinterpret_cast<u32x4 *>(gn[p] + tok * kG + 8 * ((4 * lc + q) ^ fr)) = gp[tt][p];
    }
    const int slot = (4 * ls + q) ^ (fr >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = 32 * lc + 16 * h + fr;
      const f32x4 z{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < XP; ++p) {
        const f32x4 d0 = mfma16x16x32<MG>(xp[0][p], oh[h], z), d1 = mfma16x16x32<MG>(xp[1][p], oh[h], z);
        *reinterpret_cast<u32x4 *>(xt[p] + ch * kFT + 8 * slot) =
            u32x4{pack2<MG>(d0[0], d0[1]), pack2<MG>(d0[2], d0[3]), pack2<MG>(d1[0], d1[1]), pack2<MG>(d1[2], d1[3])};
      }
#pragma unroll
      for (int p = 0; p < GP; ++p) {
        const f32x4 d0 = mfma16x16x32<MG>(gp[0][p], oh[h], z), d1 = mfma16x16x32<MG>(gp[1][p], oh[h], z);
        *reinterpret_cast<u32x4 *>(gt[p] + ch * kFT + 8 * slot) =
            u32x4{pack2<MG>(d0[0], d0[1]), pack2<MG>(d0[2], d0[3]), pack2<MG>(d1[0], d1[1]), pack2<MG>(d1[2], d1[3])};
      }
    }
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      acc[it][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_fence(acc[it][kt]);
    }
  asm volatile("s_nop 7");

  auto read_n = [&](int tt, int ks, int p) {
    const int tok = 16 * tt + fr;
    return *reinterpret_cast<const u32x4 *>(gn[p] + tok * kG + 8 * ((4 * ks + q) ^ fr));
  };
  auto read_t = [&](const uint16_t *arr, int ch, int sp) {
    return *reinterpret_cast<const u32x4 *>(arr + ch * kFT + 8 * ((4 * sp + q) ^ (fr >> 1)));
  };

  // one tile: transposes into LDS, the next-but-one tile's loads, products, dL/dx stores
  auto tile = [&](auto set, int64_t m0) {
    __syncthreads();          // the previous tile's fragments are read
    asm volatile("s_nop 7");  // before VALU reuses registers the last asm MFMAs read
    __builtin_amdgcn_sched_barrier(0);
    store_tile(set);
    if (m0 + PF * kFT < m_end) load_tile(set, m0 + PF * kFT);  // in flight for PF tiles' products
    __syncthreads();

    // dL/dx^T tiles (it: 16 rows of R', t2: 16 tokens of 32 dt ..), k over the 128 channels
    f32x4 acc2[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        acc2[it][t2] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_fence(acc2[it][t2]);
      }
    asm volatile("s_nop 7");
    // B fragment ring (step = 4 t2 + ks), filled two steps ahead: a load never
    // targets registers that the asm MFMAs just issued may still be reading
    constexpr int NB = 3;
    u32x4 bn[NB][GP];
#pragma unroll
    for (int b = 0; b < NB - 1; ++b)
#pragma unroll
      for (int p = 0; p < GP; ++p) bn[b][p] = read_n(2 * dt, b, p);
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      const int nx = step + NB - 1;
      if (nx < 8) {
#pragma unroll
        for (int p = 0; p < GP; ++p) bn[nx % NB][p] = read_n(2 * dt + (nx >> 2), nx & 3, p);
      }
      const int t2 = step >> 2, ks = step & 3;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        mfma_acc_after_valu<MX>(ar[it][ks][0], bn[step % NB][0], acc2[it][t2]);
        mfma_acc_after_valu<MX>(ar[it][ks][1], bn[step % NB][0], acc2[it][t2]);
        if constexpr (GP == 2) mfma_acc_after_valu<MX>(ar[it][ks][0], bn[step % NB][1], acc2[it][t2]);
      }
    }

    // Gram: k-step sp = tokens 32sp .. 32sp+31 of the tile
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      u32x4 a[2][XP];
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int p = 0; p < XP; ++p) a[it][p] = read_t(xt[p], 32 * gi + 16 * it + fr, sp);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        u32x4 b[GP];
#pragma unroll
        for (int p = 0; p < GP; ++p) b[p] = read_t(gt[p], 64 * gk + 16 * kt + fr, sp);
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int xp = 0; xp < XP; ++xp)
#pragma unroll
            for (int gp = 0; gp < GP; ++gp) mfma_acc_after_valu<MG>(a[it][xp], b[gp], acc[it][kt]);
      }
    }

    mfma_drain();
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) acc_fence(acc2[it][t2]);
    // lane l of tile (it, t2): token 32 dt + 16 t2 + l%16, channels 32 dr + 8(l/16) + 4it + r
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int64_t tok = m0 + 32 * dt + 16 * t2 + fr;
      if (tok < m_end) {
        const int64_t off = tok * I + g * kG + 32 * dr + 8 * q;
        const f32x4 lo4 = acc2[0][t2], hi4 = acc2[1][t2];
        if (gx_f32) {
          float *o = reinterpret_cast<float *>(gx) + off;
          __builtin_nontemporal_store(lo4, reinterpret_cast<f32x4 *>(o));
          __builtin_nontemporal_store(hi4, reinterpret_cast<f32x4 *>(o + 4));
        } else {
          const u32x4 v{pack2<XDT>(lo4[0], lo4[1]), pack2<XDT>(lo4[2], lo4[3]), pack2<XDT>(hi4[0], hi4[1]),
                        pack2<XDT>(hi4[2], hi4[3])};
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(gx) + off));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (m_begin < m_end) load_tile(Const<0>{}, m_begin);
  if constexpr (PF == 2) {
    if (m_begin + kFT < m_end) load_tile(Const<PF - 1>{}, m_begin + kFT);
    for (int64_t m0 = m_begin; m0 < m_end; m0 += 2 * kFT) {
      tile(Const<0>{}, m0);
      if (m0 + kFT >= m_end) break;
      tile(Const<PF - 1>{}, m0 + kFT);
    }
  } else {
    for (int64_t m0 = m_begin; m0 < m_end; m0 += kFT) tile(Const<0>{}, m0);
  }
  mfma_drain();
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc_fence(acc[it][kt]);

  // lane l of tile (it, kt): rows 32 gi + 16it + 4(l/16) + r, column 64 gk + 16kt + l%16
  float *out = cpart + ((int64_t)blockIdx.y * groups + g) * (kG * kG);
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(32 * gi + 16 * it + 4 * q + r) * kG + 64 * gk + 16 * kt + fr] = acc[it][kt][r];
}

// ---------------------------------------------------------------------------
// Walk kernel: rows i of C^T (columns of C) of one group, 8 per wave, four
// workgroups per group.  Lane p owns pair p of every stage (as in the forward
// rotation).  Writes dL/dcs_i and the wave's dtheta partial sums.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
bwd_walk_kernel(const float *__restrict__ cpart, int splits, int64_t I, const int16_t *__restrict__ pairs,
                const float *__restrict__ theta, const float *__restrict__ cscale, int krot, int gmask,
                float *__restrict__ gcs, float *__restrict__ tpart) {
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
// token splits: as many as keep every fused workgroup resident at once
int64_t gram_splits(int64_t tokens, int64_t I) {
  const int64_t groups = I / kG, tiles = (tokens + kFT - 1) / kFT;
  int64_t s = kGramResident / groups;
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
  const int64_t tiles = (tokens + kFT - 1) / kFT;
  L.chunk = ((tiles + L.splits - 1) / L.splits) * kFT;
  if (L.chunk == 0) L.chunk = kFT;
  L.hl_off = 0;
  L.c_off = align256((size_t)(I / kG) * kBwdMat * 2);
  L.t_off = L.c_off + align256((size_t)L.splits * (size_t)(I / kG) * kG * kG * 4);
  L.total = L.t_off + align256((size_t)kWalkParts * (size_t)krot * (size_t)(I / 2) * 4);
  return L;
}
}  // namespace

size_t rot_backward_partial_bytes(int64_t tokens, int64_t I, int krot) { return bwd_layout(tokens, I, krot).total; }

template <int XDT, int GDT>
static void launch_gram_dx(dim3 grid, hipStream_t st, const void *x, const void *g, void *gx, int gx_f32,
                           int64_t tokens, int64_t I, int64_t chunk, const uint16_t *hl, float *cpart) {
  hipLaunchKernelGGL((bwd_gram_dx_kernel<XDT, GDT>), grid, dim3(512), 0, st, x, g, gx, gx_f32, tokens, I, chunk, hl,
                     cpart);
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
  const int gm = kG - group;

  // 1. R' = diag(cs) R as H + L, rows in MFMA order
  const dim3 rgrid(groups, kG / kRowsPerBuild);
  if (dx_mdt(g_dt) == kF16)
    hipLaunchKernelGGL((bwd_rrow_kernel<kF16>), rgrid, dim3(64), 0, st, I, pairs, theta, cs, krot, gm, hl);
  else
    hipLaunchKernelGGL((bwd_rrow_kernel<kBF16>), rgrid, dim3(64), 0, st, I, pairs, theta, cs, krot, gm, hl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 2. Gram partials and dL/dx in one pass (with no tokens: one split of zeros)
  const dim3 ggrid(groups, (unsigned)L.splits);
  const int f32 = gx_dt == kF32;
  if (x_dt == kF16) {
    if (g_dt == kF32) launch_gram_dx<kF16, kF32>(ggrid, st, x, gin, gx, f32, tokens, I, L.chunk, hl, cpart);
    else launch_gram_dx<kF16, kF16>(ggrid, st, x, gin, gx, f32, tokens, I, L.chunk, hl, cpart);
  } else {
    if (g_dt == kF32) launch_gram_dx<kBF16, kF32>(ggrid, st, x, gin, gx, f32, tokens, I, L.chunk, hl, cpart);
    else launch_gram_dx<kBF16, kBF16>(ggrid, st, x, gin, gx, f32, tokens, I, L.chunk, hl, cpart);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 3. the stage walk: dL/dcs and dtheta partials
  const dim3 wgrid(groups, kG / (4 * kWalkRows));
  hipLaunchKernelGGL(bwd_walk_kernel, wgrid, dim3(256), 0, st, cpart, (int)L.splits, I, pairs, theta, cs, krot, gm,
                     gcs, tpart);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 4. dL/dtheta
  const int64_t n = (int64_t)krot * (I / 2);
  hipLaunchKernelGGL(bwd_theta_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tpart, n, gtheta);
  return hipGetLastError();
}

}  // namespace paro

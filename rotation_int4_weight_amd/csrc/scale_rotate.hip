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
#include <stdlib.h>

#include "common.hpp"
#include "launch.hpp"
#include "mx.hpp"
#include "mfma.hpp"

namespace paro {

constexpr int kRotRS = kG + 4;   // LDS row stride (floats), staggers banks across rows

template <int XDT, int ODT, int RW>
__global__ void __launch_bounds__(256)
scale_rotate_kernel(const uint16_t *__restrict__ x, void *__restrict__ xr, int64_t tokens, int64_t I,
                    const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                    const float *__restrict__ cscale, int krot, int gmask) {
  __shared__ float lds[4][RW * kRotRS];
  // all arguments in one batch of scalar loads (see decode_kernel)
  asm volatile("" ::"s"(x), "s"(xr), "s"(tokens), "s"(I), "s"(pairs), "s"(theta), "s"(cscale), "s"(krot),
               "s"(gmask));
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t m0 = ((int64_t)blockIdx.y * 4 + wave) * RW;
  if (m0 >= tokens) return;  // whole wave idle (no block-level barrier below)
  const int T = (int)((tokens - m0) < RW ? (tokens - m0) : RW);
  float *xs = lds[wave];
  const int64_t c0 = g * kG + 2 * lane;

  RotParams rp;
  rp.load(pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane, gmask);
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

  rotate_rows_lds<RW>(xs, kRotRS, rp, pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane, gmask);

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

// ---------------------------------------------------------------------------
// Tiled output for the prefill GEMM, on the matrix cores.
//
// The rotation of one 128-channel group is a fixed linear map, so
//     x_r[m][g*128 + j] = sum_i x[m][g*128 + i] * R'_g[i][j],
//     R'_g = diag(cs_g) . R_g      (R_g: the krot stages applied in order)
// (composition of linear maps: the staged result is this product exactly in
// real arithmetic).
// rot_build_kernel forms R'_g^T = R_g^T . diag(cs_g) row by row: unit row e_j
// through the transposed stages (each a Givens rotation by -theta) in reverse
// order, then times cs (the same staged code as above, fp32).  It stores R'_g
// as two matrices in the activation dtype, R' = H + L with H = rne(R') and
// L = rne(R' - H): their sum represents R' to about 2^-16 relative (bf16;
// 2^-22 for fp16), far inside the rotated-activation tolerance.
// rot_apply_kernel then computes x.H + x.L with v_mfma_f32_16x16x32 in fp32
// (x is exact in its own dtype), rounds once to the activation dtype and
// writes the tiled layout.  At 2048 tokens the build is 1/16 of the staged
// work and the rest runs on the matrix cores instead of as LDS gathers.
// ---------------------------------------------------------------------------

// hl: [group][2 (H, L)][128 (output channel, MFMA order)][128 (input channel i)],
// x dtype.  The apply kernel computes the transpose, x_r^T = R'^T . x^T, with
// H_T / L_T as the A operand: A row 4q+r (q, r < 4) of the 16-row tile 2b+h
// (b < 4, h < 2) is output channel 32b + 8q + 4h + r.  The accumulators of
// tiles 2b and 2b+1 then give each lane, for its token l%16, the channels
// 32b + 8(l/16) .. +7 in order: one 16-byte piece of the tiled layout.
constexpr int64_t kRotMatHalves = 2 * kG * kG;  // per group

constexpr int kBuildRows = 16;  // rows of H_T / L_T per one-wave workgroup

__device__ __forceinline__ int channel_of_mfma_row(int r) {
  return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

// One wave: group g = blockIdx.x, rows r0 = 16 * blockIdx.y .. r0+15 of H_T and
// L_T (output channels j = channel_of_mfma_row(r)).  Each row is written as
// one coalesced 256-byte store per matrix.
template <int XDT>
__global__ void __launch_bounds__(64)
rot_build_kernel(int64_t I, const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                 const float *__restrict__ cscale, int krot, int gmask, uint16_t *__restrict__ hl) {
  constexpr int RW = kBuildRows;
  __shared__ float xs[RW * kRotRS];
  const int lane = lane_id();
  const int64_t g = blockIdx.x;
  const int r0 = blockIdx.y * RW;
  const int16_t *pairs_g = pairs + g * kG;
  const float *theta_g = theta + g * kPairs;

  // parameters of the last kStageRegs stages (applied first), issued up front
  uint32_t pw[kStageRegs];
  float th[kStageRegs];
#pragma unroll
  for (int u = 0; u < kStageRegs; ++u) {
    const int t = krot - 1 - u >= 0 ? krot - 1 - u : 0;
    pw[u] = load_pair_word(pairs_g, I, t, lane, gmask);
    th[u] = theta_g[(int64_t)t * (I / 2) + lane];
  }
  const float2 cs2 = *reinterpret_cast<const float2 *>(cscale + g * kG + 2 * lane);

#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const int j = channel_of_mfma_row(r0 + m);
    xs[m * kRotRS + 2 * lane] = 2 * lane == j ? 1.0f : 0.0f;
    xs[m * kRotRS + 2 * lane + 1] = 2 * lane + 1 == j ? 1.0f : 0.0f;
  }
  wave_lds_sync();

#pragma unroll
  for (int u = 0; u < kStageRegs; ++u) {
    if (u < krot) {
      float c, sn;
      __sincosf(th[u], &sn, &c);
      rotate_stage<RW>(xs, kRotRS, pw[u], c, -sn);
    }
  }
  for (int t = krot - 1 - kStageRegs; t >= 0; --t) {
    const uint32_t w = load_pair_word(pairs_g, I, t, lane, gmask);
    float c, sn;
    __sincosf(theta_g[(int64_t)t * (I / 2) + lane], &sn, &c);
    rotate_stage<RW>(xs, kRotRS, w, c, -sn);
  }

  // xs[m][i] * cs[i] = R'[i][j_m]: lane p holds input channels 2p, 2p+1
  uint32_t *hrow = reinterpret_cast<uint32_t *>(hl + g * kRotMatHalves + (int64_t)r0 * kG) + lane;
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    const float v0 = xs[m * kRotRS + 2 * lane] * cs2.x, v1 = xs[m * kRotRS + 2 * lane + 1] * cs2.y;
    const uint32_t hb = pack2<XDT>(v0, v1);
    const float e0 = v0 - act_to_f32<XDT>(hb & 0xffffu), e1 = v1 - act_to_f32<XDT>(hb >> 16);  // exact
    hrow[m * (kG / 2)] = hb;
    hrow[(kG + m) * (kG / 2)] = pack2<XDT>(e0, e1);
  }
}

// One workgroup: group g = blockIdx.x, token rows [R*blockIdx.y, +R) with
// R = 16 * wg_tiles (apply_rows below); each wave takes batches of 4 row
// tiles (64 rows) and fetches the next batch's x while it computes the
// current one.  LDS holds H_T and L_T of the group (row stride 136 halves:
// the 16-byte fragment reads of 16 lanes spread over the banks).
constexpr int kHS = kG + 8;
// default token rows per workgroup of the MXFP4 variant: with its epilogue
// (VALU-heavy) two workgroups per CU overlap it with the other's products:
// 42.1 us at 512 rows against 56.9 us at 1024
constexpr int kApplyRowsMx = 512;
constexpr int kApplyCUs = 256;  // compute units of an MI355X (one plain-apply workgroup each)
constexpr int kApplyTiles = 4;  // row tiles per wave and batch

// X staging of the plain apply (MX = false): a wave's next batch of 64 token
// rows x 128 channels moves global -> LDS in 16 DMA loads of 4 whole
// 256-byte row pieces each (lane l: row l%4, 16-byte chunk l/4), instead
// of 16 register loads of 16 rows x 64 bytes: wider pieces stream faster
// (about 12 % on 2048 x 14336).  Load q lands in block q of the wave's
// region (1 KB + 64 bytes of padding), so that a fragment read (16 rows of
// one 16-byte chunk) touches 16 distinct 16-byte bank groups.
constexpr int kXBlk = (1024 + 64) / 2;  // halves per staged load block
// One 1 KB global -> LDS load: lane l's 16 bytes at voff + soff land at
// lds + 16 l.  (A plain device function: inside a kernel template the
// builtin would keep the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void apply_dma_1k(__amdgpu_buffer_rsrc_t r, uint16_t *lds, uint32_t voff, uint32_t soff) {
  typedef __attribute__((address_space(3))) void *lds_ptr;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
}

// MX = true: instead of the tiled X_r, each row's 32-channel blocks are
// quantized to MXFP4 in the epilogue (codes [tokens][I/2], E8M0 scales
// [tokens][I/32]): a lane holds 8 consecutive channels of a block, and the
// block's other 24 are in lanes l ^ 16, l ^ 32, l ^ 48 (same token).
template <int XDT, bool MX>
__global__ void __launch_bounds__(256, MX ? 2 : 1)  // the plain apply's x staging fills the LDS of one
rot_apply_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ xt, int64_t tokens, int64_t I,
                 const uint16_t *__restrict__ hl, uint8_t *__restrict__ mx_codes, uint8_t *__restrict__ mx_scales,
                 int wg_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t hlds[2 * kG * kHS];
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int64_t g = blockIdx.x;
  const int64_t mt_end = tiled_rows(tokens) / 16;  // row tiles of the tiled buffer
  const int64_t mt_first = (int64_t)blockIdx.y * wg_tiles;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  const uint32_t lane_off = (uint32_t)((fr * I + fk) * 2);

  // x fragments (B operand: token l%16, input channels 8(l/16)..+7 of k-step
  // ks) of the batch starting at row tile mt0; raw buffer over its 64 rows, so
  // rows past the last token read as zeros.
  auto load_x = [&](int64_t mt0, u32x4 (&xf)[kApplyTiles][4]) {
    const int64_t row0 = mt0 * 16;
    const int64_t rows = tokens - row0 < 64 ? tokens - row0 : 64;
    const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x + row0 * I + g * kG, rows > 0 ? (uint32_t)(rows * I * 2) : 0u);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < kApplyTiles; ++t)
        xf[t][ks] = __builtin_amdgcn_raw_buffer_load_b128(xr, lane_off, (int)((t * 16 * I + ks * 32) * 2), 0);
  };

  int64_t mt0 = mt_first + wave * kApplyTiles;
  u32x4 xf[kApplyTiles][4];
  // plain apply: the staged batch's region of this wave, the DMA lane offset
  // and the lane's fragment offset in the region (row 16t + fr lies in block
  // 4t + fr/4 at row position fr%4; chunk 4ks + l/16)
  __shared__ __attribute__((aligned(16))) uint16_t xlds[MX ? 1 : 4][MX ? 8 : 16 * kXBlk];
  uint16_t *xw = xlds[MX ? 0 : wave];
  const uint32_t dma_voff = (uint32_t)(((lane & 3) * I + 8 * (lane >> 2)) * 2);
  const int xf_off = (fr >> 2) * kXBlk + 32 * (lane >> 4) + 8 * (fr & 3);
  auto dma_x = [&](int64_t mt) {
    const int64_t row0 = mt * 16;
    const int64_t rows = tokens - row0 < 64 ? tokens - row0 : 64;
    const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x + row0 * I + g * kG, rows > 0 ? (uint32_t)(rows * I * 2) : 0u);
#pragma unroll
    for (int q = 0; q < 16; ++q) apply_dma_1k(xr, xw + q * kXBlk, dma_voff, (uint32_t)(4 * q * I * 2));
  };
  auto read_x = [&]() {
#pragma unroll
    for (int t = 0; t < kApplyTiles; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        xf[t][ks] = *reinterpret_cast<const u32x4 *>(xw + xf_off + 4 * t * kXBlk + 128 * ks);
  };
  if (mt0 < mt_end && mt0 < mt_first + wg_tiles) {
    if constexpr (MX)
      load_x(mt0, xf);
    else
      dma_x(mt0);
  }

  // H_T, L_T of the group into LDS: 256 rows x 16 chunks of 16 bytes (16 per
  // thread, in two halves so that the x fragments in flight stay in registers)
  const uint16_t *hg = hl + g * kRotMatHalves;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = threadIdx.x + 256 * (8 * half + u);  // chunk: matrix row c/16 (of 256), part c%16
      const u32x4 v = *reinterpret_cast<const u32x4 *>(hg + (int64_t)c * 8);
      *reinterpret_cast<u32x4 *>(hlds + (c >> 4) * kHS + (c & 15) * 8) = v;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if constexpr (!MX) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the first batch has landed in LDS
    read_x();
  }

  constexpr int kStride = 4 * kApplyTiles;  // row tiles per batch of the workgroup
  for (; mt0 < mt_end && mt0 < mt_first + wg_tiles; mt0 += kStride) {
    const int64_t next = mt0 + kStride;
    const bool more = next < mt_end && next < mt_first + wg_tiles;
    if constexpr (!MX) {
      // the fragment reads of this batch are done before its region is
      // rewritten with the next batch
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (more) dma_x(next);
    }
    f32x4 acc[kApplyTiles][8];
#pragma unroll
    for (int t = 0; t < kApplyTiles; ++t)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        acc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_fence(acc[t][ct]);
      }
    asm volatile("s_nop 7");  // accumulator writes -> first MFMA
    // 64 steps (k-step ks, channel tile ct, H or L): one 16-byte LDS read of
    // the A fragment, issued two steps ahead, and 4 MFMAs (one per row tile)
    auto read_a = [&](int step) {
      const int ks = step >> 4, ct = (step >> 1) & 7, hlm = step & 1;
      return *reinterpret_cast<const u32x4 *>(hlds + (hlm * kG + ct * 16 + fr) * kHS + ks * 32 + fk);
    };
    u32x4 ar[3];
    ar[0] = read_a(0);
    ar[1] = read_a(1);
#pragma unroll
    for (int step = 0; step < 64; ++step) {
      const int ks = step >> 4, ct = (step >> 1) & 7;
      if (step + 2 < 64) ar[(step + 2) % 3] = read_a(step + 2);
#pragma unroll
      for (int t = 0; t < kApplyTiles; ++t) mfma_acc<XDT>(ar[step % 3], xf[t][ks], acc[t][ct]);
      if (MX && (step & 15) == 15 && more) {  // k-step ks consumed: fetch the next batch's fragments
        const int64_t row0 = next * 16;
        const int64_t rows = tokens - row0 < 64 ? tokens - row0 : 64;
        const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x + row0 * I + g * kG, (uint32_t)(rows * I * 2));
#pragma unroll
        for (int t = 0; t < kApplyTiles; ++t)
          xf[t][ks] = __builtin_amdgcn_raw_buffer_load_b128(xr, lane_off, (int)((t * 16 * I + ks * 32) * 2), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_drain();
#pragma unroll
    for (int t = 0; t < kApplyTiles; ++t)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc_fence(acc[t][ct]);
    if constexpr (!MX) {
      if (more) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next batch has landed
        read_x();
      }
    }
    // lane l, tile t, 32-channel block b: token l%16, channels 32b + 8(l/16) .. +7.
    if constexpr (MX) {
#pragma unroll
      for (int t = 0; t < kApplyTiles; ++t) {
        const int64_t tok = (mt0 + t) * 16 + fr;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x4 lo = acc[t][2 * b], hi = acc[t][2 * b + 1];
          const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          float am = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
          am = fmaxf(am, __shfl_xor(am, 16));
          am = fmaxf(am, __shfl_xor(am, 32));
          const int biased = mx_block_exponent(am);
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            word |= e2m1_pair(mx_scaled(v[e], biased), mx_scaled(v[e + 1], biased)) << (4 * e);
          if (tok < tokens) {
            *reinterpret_cast<uint32_t *>(mx_codes + tok * (I / 2) + g * (kG / 2) + 16 * b + (fk >> 1)) = word;
            if (fk == 0) mx_scales[tok * (I / 32) + g * 4 + b] = (uint8_t)biased;
          }
        }
      }
      continue;
    }
    // Streaming (non-temporal) stores: X_r is not read again by this kernel,
    // and keeping it out of the caches leaves them to the x stream (measured
    // a third faster than ordinary stores).
#pragma unroll
    for (int t = 0; t < kApplyTiles; ++t) {
      if (mt0 + t >= mt_end) break;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 lo = acc[t][2 * b], hi = acc[t][2 * b + 1];
        const u32x4 v{pack2<XDT>(lo[0], lo[1]), pack2<XDT>(lo[2], lo[3]), pack2<XDT>(hi[0], hi[1]),
                      pack2<XDT>(hi[2], hi[3])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(xt + ((mt0 + t) * (I / 32) + g * 4 + b) * 512 + lane * 8));
      }
    }
  }
}

size_t rot_mat_bytes(int64_t I) { return (size_t)(I / kG) * (size_t)kRotMatHalves * 2; }

hipError_t launch_rot_build(int x_dt, int64_t I, const int16_t *pairs, const float *theta, const float *cs,
                            int krot, int group, uint16_t *hl, hipStream_t st) {
  const dim3 grid((unsigned)(I / kG), kG / kBuildRows);
  const int gm = kG - group;
  if (x_dt == kF16)
    hipLaunchKernelGGL((rot_build_kernel<kF16>), grid, dim3(64), 0, st, I, pairs, theta, cs, krot, gm, hl);
  else
    hipLaunchKernelGGL((rot_build_kernel<kBF16>), grid, dim3(64), 0, st, I, pairs, theta, cs, krot, gm, hl);
  return hipGetLastError();
}

// token rows per apply workgroup; tuning override PARO_APPLY_ROWS (256, 512,
// 1024, 2048 or 4096), read once per process.  Without it: the MXFP4
// variant (two workgroups per CU) starts from its default and halves it
// (down to 256) while the launch would have fewer than 192 workgroups, so
// narrow layers still spread over the chip; the plain apply (one workgroup
// per CU, its LDS holds the x staging) takes the fewest rows, from 256 up,
// whose grid fits the 256 CUs in one round (2048 x 14336: 1024 rows, 224
// workgroups; 4096 x 14336: 2048 rows, 224 workgroups, against 448 in two
// rounds at 1024).
static int apply_rows(int dflt, int64_t tokens, int64_t I, bool one_per_cu) {
  static const int r = [] {
    const char *v = getenv("PARO_APPLY_ROWS");
    const int n = (v && *v) ? atoi(v) : 0;
    return (n == 256 || n == 512 || n == 1024 || n == 2048 || n == 4096) ? n : 0;
  }();
  if (r) return r;
  auto grid = [&](int rows) { return (I / kG) * ((tiled_rows(tokens) + rows - 1) / rows); };
  if (one_per_cu) {
    int rows = 256;
    while (rows < 4096 && grid(rows) > kApplyCUs) rows *= 2;
    return rows;
  }
  int rows = dflt;
  while (rows > 256 && grid(rows) < 192) rows /= 2;
  return rows;
}

hipError_t launch_rot_apply(const uint16_t *x, int x_dt, uint16_t *xt, int64_t tokens, int64_t I,
                            const uint16_t *hl, hipStream_t st) {
  const int rows = apply_rows(0, tokens, I, true);
  const dim3 grid((unsigned)(I / kG), (unsigned)((tiled_rows(tokens) + rows - 1) / rows));
  if (x_dt == kF16)
    hipLaunchKernelGGL((rot_apply_kernel<kF16, false>), grid, dim3(256), 0, st, x, xt, tokens, I, hl, nullptr,
                       nullptr, rows / 16);
  else
    hipLaunchKernelGGL((rot_apply_kernel<kBF16, false>), grid, dim3(256), 0, st, x, xt, tokens, I, hl, nullptr,
                       nullptr, rows / 16);
  return hipGetLastError();
}

hipError_t launch_rot_apply_mx(const uint16_t *x, int x_dt, int64_t tokens, int64_t I, const uint16_t *hl,
                               uint8_t *codes, uint8_t *scales, hipStream_t st) {
  if (tokens == 0) return hipSuccess;
  const int rows = apply_rows(kApplyRowsMx, tokens, I, false);
  const dim3 grid((unsigned)(I / kG), (unsigned)((tiled_rows(tokens) + rows - 1) / rows));
  if (x_dt == kF16)
    hipLaunchKernelGGL((rot_apply_kernel<kF16, true>), grid, dim3(256), 0, st, x, nullptr, tokens, I, hl, codes,
                       scales, rows / 16);
  else
    hipLaunchKernelGGL((rot_apply_kernel<kBF16, true>), grid, dim3(256), 0, st, x, nullptr, tokens, I, hl, codes,
                       scales, rows / 16);
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

// ---------------------------------------------------------------------------
// One rotation group over the whole row (group_size -1, i.e. G = I).
//
// "ParoQuant" wiki, Concepts / Pairwise Givens rotations: group_size -1 is one
// group of all in_features channels, so a stage's pairs may join any two
// channels of the row and the 128-channel blocks above do not apply (nor
// does the dense per-block form).  A workgroup holds R scaled rows of x in
// LDS (fp32, R * I * 4 <= 64 KB); at each stage its threads take the I/2
// pairs in turn and apply them to all R rows with the same fp32 operations
// as rotate_stage; a barrier separates the stages.  Pair indices past the
// row are read as 0, so a bad schedule cannot leave the row's LDS.  The
// result goes out row-major (xr dtype) or, TILED, in the prefill GEMM's
// tiled layout: the grid then covers every 16-row tile of it, pad rows
// (zero in, zero out) included, with R dividing 16.
// ---------------------------------------------------------------------------
constexpr int kFullThreads = 256;

template <int XDT, int ODT, bool TILED>
__global__ void __launch_bounds__(kFullThreads)
scale_rotate_full_kernel(const uint16_t *__restrict__ x, void *__restrict__ xr, int64_t tokens, int64_t I, int R,
                         const int16_t *__restrict__ pairs, const float *__restrict__ theta,
                         const float *__restrict__ cscale, int krot) {
  extern __shared__ __attribute__((aligned(16))) float rows[];  // [R][I]
  // all arguments in one batch of scalar loads (see decode_kernel)
  asm volatile("" ::"s"(x), "s"(xr), "s"(tokens), "s"(I), "s"(R), "s"(pairs), "s"(theta), "s"(cscale), "s"(krot));
  const int64_t m0 = (int64_t)blockIdx.x * R;
  const int64_t half = I / 2;
  for (int64_t e = threadIdx.x; e < R * half; e += kFullThreads) {
    const int r = (int)(e / half);
    const int64_t k = 2 * (e - r * half);
    float v0 = 0.0f, v1 = 0.0f;
    if (m0 + r < tokens) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(x + (m0 + r) * I + k);
      v0 = act_to_f32<XDT>(w & 0xffffu) * cscale[k];
      v1 = act_to_f32<XDT>(w >> 16) * cscale[k + 1];
    }
    rows[r * I + k] = v0;
    rows[r * I + k + 1] = v1;
  }
  __syncthreads();
  for (int t = 0; t < krot; ++t) {
    const int16_t *pt = pairs + (int64_t)t * I;
    const float *tt = theta + (int64_t)t * half;
    for (int64_t p = threadIdx.x; p < half; p += kFullThreads) {
      const uint32_t pw = *reinterpret_cast<const uint32_t *>(pt + 2 * p);
      const int64_t ia = pw & 0xffffu, ib = pw >> 16;
      const int64_t a = ia < I ? ia : 0, b = ib < I ? ib : 0;
      float c, sn;
      __sincosf(tt[p], &sn, &c);
      for (int r = 0; r < R; ++r) {
        const float va = rows[r * I + a], vb = rows[r * I + b];
        rows[r * I + a] = __builtin_fmaf(va, c, vb * sn);
        rows[r * I + b] = __builtin_fmaf(vb, c, -(va * sn));
      }
    }
    __syncthreads();
  }
  if constexpr (TILED) {
    // 8 consecutive channels of one row per thread and pass: one 16-byte piece
    const int64_t chunks = I / 8;
    for (int64_t e = threadIdx.x; e < R * chunks; e += kFullThreads) {
      const int r = (int)(e / chunks);
      const int64_t c = e - r * chunks, k = 8 * c, m = m0 + r;
      const float *v = rows + r * I + k;
      const u32x4 q{pack2<ODT>(v[0], v[1]), pack2<ODT>(v[2], v[3]), pack2<ODT>(v[4], v[5]), pack2<ODT>(v[6], v[7])};
      const int64_t idx = ((m / 16) * (I / 32) + k / 32) * 512 + (((k % 32) / 8) * 16 + m % 16) * 8;
      *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(xr) + idx) = q;
    }
  } else {
    for (int64_t e = threadIdx.x; e < R * half; e += kFullThreads) {
      const int r = (int)(e / half);
      const int64_t k = 2 * (e - r * half);
      if (m0 + r >= tokens) continue;
      const float v0 = rows[r * I + k], v1 = rows[r * I + k + 1];
      const int64_t o = (m0 + r) * I + k;
      if constexpr (ODT == kF32)
        *reinterpret_cast<float2 *>(reinterpret_cast<float *>(xr) + o) = make_float2(v0, v1);
      else
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(xr) + o) = pack2<ODT>(v0, v1);
    }
  }
}

int full_row_rows(int64_t I) {
  int r = 16;
  while (r > 1 && (int64_t)r * I * 4 > kFullRowLdsBytes) r /= 2;
  return r;
}

template <int XDT, int ODT, bool TILED>
static hipError_t launch_full_t(const uint16_t *x, void *xr, int64_t tokens, int64_t I, const int16_t *pairs,
                                const float *theta, const float *cs, int krot, hipStream_t st) {
  const int R = full_row_rows(I);
  const int64_t rows = TILED ? tiled_rows(tokens) : tokens;
  const dim3 grid((unsigned)((rows + R - 1) / R));
  hipLaunchKernelGGL((scale_rotate_full_kernel<XDT, ODT, TILED>), grid, dim3(kFullThreads),
                     (size_t)R * I * sizeof(float), st, x, xr, tokens, I, R, pairs, theta, cs, krot);
  return hipGetLastError();
}

hipError_t launch_scale_rotate_full(const uint16_t *x, int x_dt, void *xr, int xr_dt, bool tiled, int64_t tokens,
                                    int64_t I, const int16_t *pairs, const float *theta, const float *cs, int krot,
                                    hipStream_t st) {
  if (tokens == 0) return hipSuccess;
  if (tiled) {  // the tiled layout holds the activation dtype
    if (x_dt == kF16) return launch_full_t<kF16, kF16, true>(x, xr, tokens, I, pairs, theta, cs, krot, st);
    return launch_full_t<kBF16, kBF16, true>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  }
  if (x_dt == kF16) {
    if (xr_dt == kF16) return launch_full_t<kF16, kF16, false>(x, xr, tokens, I, pairs, theta, cs, krot, st);
    if (xr_dt == kBF16) return launch_full_t<kF16, kBF16, false>(x, xr, tokens, I, pairs, theta, cs, krot, st);
    return launch_full_t<kF16, kF32, false>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  }
  if (xr_dt == kF16) return launch_full_t<kBF16, kF16, false>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  if (xr_dt == kBF16) return launch_full_t<kBF16, kBF16, false>(x, xr, tokens, I, pairs, theta, cs, krot, st);
  return launch_full_t<kBF16, kF32, false>(x, xr, tokens, I, pairs, theta, cs, krot, st);
}

template <int XDT, int ODT, int RW>
static hipError_t launch_rot_rw(const uint16_t *x, void *xr, int64_t tokens, int64_t I, const int16_t *pairs,
                                const float *theta, const float *cs, int krot, int gm, hipStream_t st) {
  const int64_t per_block = 4 * RW;
  dim3 grid((unsigned)(I / kG), (unsigned)((tokens + per_block - 1) / per_block));
  hipLaunchKernelGGL((scale_rotate_kernel<XDT, ODT, RW>), grid, dim3(256), 0, st, x, xr, tokens, I, pairs,
                     theta, cs, krot, gm);
  return hipGetLastError();
}

template <int XDT, int ODT>
static hipError_t launch_rot(const uint16_t *x, void *xr, int64_t tokens, int64_t I, const int16_t *pairs,
                             const float *theta, const float *cs, int krot, int gm, hipStream_t st) {
  // up to 16 tokens: one row per wave (the chain of dependent LDS stages is
  // the kernel's critical path; 16 tokens x 4096 channels: 4.1 us at four
  // rows per wave)
  if (tokens <= 16) return launch_rot_rw<XDT, ODT, 1>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
  if (tokens <= 64) return launch_rot_rw<XDT, ODT, 4>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
  return launch_rot_rw<XDT, ODT, 16>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
}

hipError_t launch_scale_rotate(const uint16_t *x, int x_dt, void *xr, int xr_dt, int64_t tokens, int64_t I,
                               const int16_t *pairs, const float *theta, const float *cs, int krot,
                               int group, hipStream_t st) {
  const int gm = kG - group;
  if (x_dt == kF16) {
    if (xr_dt == kF16) return launch_rot<kF16, kF16>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
    if (xr_dt == kBF16) return launch_rot<kF16, kBF16>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
    return launch_rot<kF16, kF32>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
  }
  if (xr_dt == kF16) return launch_rot<kBF16, kF16>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
  if (xr_dt == kBF16) return launch_rot<kBF16, kBF16>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
  return launch_rot<kBF16, kF32>(x, xr, tokens, I, pairs, theta, cs, krot, gm, st);
}

}  // namespace paro

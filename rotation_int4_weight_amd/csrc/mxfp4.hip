// mxfp4.hip - four-bit activations after the rotation (the W4A4 extension's
// MXFP4 variant; "ParoQuant" blog, Bits and formats) on the CDNA4 block-scaled
// FP4 matrix cores.
//
//   y = MX(x . D^-1 . R) . MX(W . D . R)^T + b
//
// MX(.) is the OCP microscaling format along the input channels: blocks of 32
// consecutive values share an E8M0 scale 2^(b - 127) with
// b = floor(log2 max|v|) - 2 + 127 (0 for an all-zero block), and each value
// is the E2M1 number nearest to v / 2^(b - 127) (ties to the even code,
// clamped at 6; zero stored as +0).  Codes: [rows][I/2] bytes, element 2j in
// the low nibble of byte j; scales: [rows][I/32] bytes.
//
// mx_quant_kernel rotates weight rows of one 128-channel block in LDS with the
// staged rotation (fp32, W divided by cs) and quantizes them: lane p holds
// channels 2p, 2p+1, a block of 32 channels is 16 lanes, so its max is four
// lane shuffles away.  Activations are quantized in the epilogue of the dense
// rotation on the matrix cores (rot_apply_kernel<., true>).
//
// mx_gemm_kernel runs v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 A and B: lane
// l supplies row (column) l%16 and the 32 elements of K block l/16 of a
// 128-wide k step, 16 bytes of the row-major codes (staged through LDS), with
// the E8M0 scale of exactly that 32-element block; the 16x16 fp32 result has
// row 4(l/16)+r, column l%16 in register r.  (The order of the 32 elements
// inside a lane's block does not matter as long as A and B agree.)
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "mx.hpp"

namespace paro {

constexpr int kMxRS = kG + 4;  // LDS row stride (floats)

template <int DT>
__device__ __forceinline__ float2 load_pair_any(const void *p, int64_t idx) {
  if constexpr (DT == kF32) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(p) + idx);
  } else {
    const uint32_t b = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(p) + idx);
    return float2{act_to_f32<DT>(b & 0xffffu), act_to_f32<DT>(b >> 16)};
  }
}

// rows [rows][I] (x dtype, or the weight's dtype); WEIGHT: divide by cs
template <int DT, bool WEIGHT>
__global__ void __launch_bounds__(256)
mx_quant_kernel(const void *__restrict__ src, int64_t rows, int64_t I, const int16_t *__restrict__ pairs,
                const float *__restrict__ theta, const float *__restrict__ cscale, int krot, int gmask,
                uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  constexpr int RW = 16;
  __shared__ float lds[4][RW * kMxRS];
  const int lane = lane_id(), wave = wave_id();
  const int64_t g = blockIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * 64 + wave * RW;
  if (r0 >= rows) return;  // wave-uniform; no workgroup barrier below
  float *xs = lds[wave];

  RotParams rp;
  rp.load(pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane, gmask);
  const float2 csv = *reinterpret_cast<const float2 *>(cscale + g * kG + 2 * lane);
#pragma unroll
  for (int m = 0; m < RW; ++m) {
    float2 v{0.f, 0.f};
    if (r0 + m < rows) v = load_pair_any<DT>(src, (r0 + m) * I + g * kG + 2 * lane);
    xs[m * kMxRS + 2 * lane] = WEIGHT ? v.x / csv.x : v.x * csv.x;
    xs[m * kMxRS + 2 * lane + 1] = WEIGHT ? v.y / csv.y : v.y * csv.y;
  }
  wave_lds_sync();
  rotate_rows_lds<RW>(xs, kMxRS, rp, pairs + g * kG, I, theta + g * kPairs, I / 2, krot, lane, gmask);

#pragma unroll
  for (int m = 0; m < RW; ++m) {
    if (r0 + m >= rows) break;
    const float v0 = xs[m * kMxRS + 2 * lane], v1 = xs[m * kMxRS + 2 * lane + 1];
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));  // the 16 lanes of a block
    const int biased = mx_block_exponent(amax);
    const uint32_t byte = e2m1_pair(mx_scaled(v0, biased), mx_scaled(v1, biased));
    codes[(r0 + m) * (I / 2) + g * kPairs + lane] = (uint8_t)byte;
    if ((lane & 15) == 0) scales[(r0 + m) * (I / 32) + g * 4 + (lane >> 4)] = (uint8_t)biased;
  }
}

// c += A . B on one 16x16 tile with FP4 (E2M1) A and B and their E8M0 block
// scales, c tied to an AGPR quadruple (as mfma_acc: no accumulator moves
// between loop iterations).  The compiler does not see this as an MFMA: the
// scale operands are computed by VALU some instructions earlier and separated
// from the first MFMA by s_nop, and results are read only after mfma_drain.
__device__ __forceinline__ void mfma_fp4(const u32x4 &a, const u32x4 &b, uint32_t sa, uint32_t sb, f32x4 &c) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
               : "+a"(c)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// y[m][n] = sum_k A[m][k] W[n][k] (+ bias[n]).  A workgroup of 8 waves takes
// a 128 x 256 tile (waves 2 x 4, 64 x 64 each: 4 x 4 MFMA tiles) over stages
// of 256 k (two 128-wide MFMA steps).  Each stage's A and W code panels (128
// and 256 rows x 128 bytes: whole cache lines) and their two scale dwords per
// row go through LDS once per workgroup, loaded straight into LDS (no
// register staging, no LDS store instructions) into a ring of three stage
// buffers, two stages ahead of the products, with one barrier per stage.
// 16-byte chunks are XOR-swizzled by row, so that the fragment reads of 16
// rows cover all banks.  Workgroups run M-fastest in XCD-local order, so the
// M tiles that share a weight panel meet in one L2.
constexpr int kMxBM = 128, kMxBN = 256, kMxRow = 128;  // LDS row pitch (bytes): one 128-byte code line
// 16-byte chunk c of row r sits at slot c ^ ((r / 2) % 8): the fragment read
// of 16 rows at one chunk covers all 64 banks
__device__ __forceinline__ int mx_slot(int row, int c) { return row * kMxRow + 16 * (c ^ ((row >> 1) & 7)); }
constexpr int kMxA = kMxBM * kMxRow, kMxW = kMxBN * kMxRow;
constexpr int kMxS = 4096;                  // scales: two dwords per row (3 KB) and 1 KB of padding
constexpr int kMxBuf = kMxA + kMxW + kMxS;  // one stage
constexpr int kMxStages = 3;                // LDS ring: 156 KB
constexpr int kMxDma = 8;                   // direct-to-LDS loads per wave and stage
static_assert(kMxDma == 8, "the stage wait below is written as vmcnt(8)");

template <int N>
struct MxConst {
  static constexpr int value = N;
};

template <int ODT>
__global__ void __launch_bounds__(512)
mx_gemm_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t M,
               const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, int64_t N, int64_t K,
               const uint16_t *__restrict__ bias, void *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMxStages][kMxBuf];
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int m_tiles = (int)((M + kMxBM - 1) / kMxBM);
  const int lwg = xcd_local_order((int)blockIdx.x, (int)gridDim.x);
  const int64_t mt0 = (int64_t)__builtin_amdgcn_readfirstlane(lwg % m_tiles) * kMxBM;
  const int64_t nt0 = (int64_t)__builtin_amdgcn_readfirstlane(lwg / m_tiles) * kMxBN;
  const int wm = wave >> 2, wn = wave & 3;  // wave's 64 x 64 sub-tile
  const int fr = lane & 15, q = lane >> 4;
  const int64_t kb = K / 2, ks = K / 32;
  const int64_t ksteps = K / 128, nstages = (ksteps + 1) / 2;
  const __amdgpu_buffer_rsrc_t ra = raw_rsrc(ac, (uint32_t)(M * kb));
  const __amdgpu_buffer_rsrc_t rw = raw_rsrc(wc, (uint32_t)(N * kb));
  const __amdgpu_buffer_rsrc_t rsa = raw_rsrc(as, (uint32_t)(M * ks));
  const __amdgpu_buffer_rsrc_t rsw = raw_rsrc(ws, (uint32_t)(N * ks));

  // Direct global -> LDS loads of one stage (buffer_load ... lds: lane l's 16
  // (4) bytes land at the window base + 16l (4l)).  A wave fills 1 KB windows
  // of 8 code rows: lane l takes slot l of the window, i.e. row l/8 and the
  // global chunk whose swizzled slot is l%8.  A: windows wave, wave + 8 (128
  // rows); W: wave + 8u, u < 4 (256 rows).  Scales: 256-byte windows of 32
  // rows (two dwords each), wave and wave + 8 of 16: windows 0..3 are A's
  // rows, 4..11 W's, 12..15 re-read row 0 into the padding, so every wave
  // issues kMxDma loads per stage.  Chunks past the end of K (an odd last
  // step) are re-read in bounds and unused.
  uint32_t a_off[2], w_off[4], s_off[2];
  bool s_isa[2], s_hi[2];
  const int wrow = lane >> 3, wslot = lane & 7;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 8 * (wave + 8 * u) + wrow;
    a_off[u] = (uint32_t)((mt0 + row) * kb + 16 * (wslot ^ ((row >> 1) & 7)));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 8 * (wave + 8 * u) + wrow;
    w_off[u] = (uint32_t)((nt0 + row) * kb + 16 * (wslot ^ ((row >> 1) & 7)));
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int win = wave + 8 * u, d = 64 * win + lane;  // dword d of the scale region
    const int row = win < 12 ? d >> 1 : 0, half = win < 12 ? d & 1 : 0;
    s_isa[u] = row < kMxBM;
    s_hi[u] = half == 1;
    s_off[u] = (uint32_t)((s_isa[u] ? (mt0 + row) : (nt0 + row - kMxBM)) * ks + 4 * half);
  }
  typedef __attribute__((address_space(3))) void *lds_ptr;
  auto dma = [&](int buf, int64_t st) {
    const bool hi_ok = 2 * st + 1 < ksteps;
    const uint32_t cb = (uint32_t)(st * 128);
    uint8_t *b = lds[buf];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 8 * (wave + 8 * u) + wrow, c = wslot ^ ((row >> 1) & 7);
      const uint32_t o = a_off[u] + cb - ((c >= 4 && !hi_ok) ? 64u : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(b + 1024 * (wave + 8 * u)), 16, o, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 8 * (wave + 8 * u) + wrow, c = wslot ^ ((row >> 1) & 7);
      const uint32_t o = w_off[u] + cb - ((c >= 4 && !hi_ok) ? 64u : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(b + kMxA + 1024 * (wave + 8 * u)), 16, o, 0, 0, 0);
    }
    const uint32_t sb = (uint32_t)(st * 8);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // the second dword of a row is the step's second half: the first one again past K
      const uint32_t o = s_off[u] + sb - ((!hi_ok && s_hi[u]) ? 4u : 0u);
      lds_ptr dst = (lds_ptr)(b + kMxA + kMxW + 256 * (wave + 8 * u));
      if (s_isa[u]) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, dst, 4, o, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, dst, 4, o, 0, 0, 0);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_fence(acc[i][j]);
    }
  asm volatile("s_nop 7");

  auto compute = [&](int buf, int h) {  // the 128-wide step h (0, 1) of the stage in buffer buf
    const uint8_t *b = lds[buf];
    u32x4 fa[4], fw[4];
    uint32_t sca[4], scw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ar = wm * 64 + 16 * i + fr, wr = wn * 64 + 16 * i + fr;
      fa[i] = *reinterpret_cast<const u32x4 *>(b + mx_slot(ar, 4 * h + q));
      fw[i] = *reinterpret_cast<const u32x4 *>(b + kMxA + mx_slot(wr, 4 * h + q));
      sca[i] = (*reinterpret_cast<const uint32_t *>(b + kMxA + kMxW + 8 * ar + 4 * h) >> (8 * q)) & 0xffu;
      scw[i] = (*reinterpret_cast<const uint32_t *>(b + kMxA + kMxW + 8 * (kMxBM + wr) + 4 * h) >> (8 * q)) & 0xffu;
    }
    // the scale operands come from VALU: padding before the asm MFMAs read them
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_fp4(fa[i], fw[j], sca[i], scw[j], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // stage s in LDS buffer s % 3: its loads were issued two stages earlier.
  // Each stage waits for this wave's loads of the stage (the next stage's
  // kMxDma stay in flight), then one barrier makes every wave's loads visible
  // and orders the refill of buffer (s + 2) % 3 (read by stage s - 1) after
  // every wave's products of stage s - 1.
  dma(0, 0);
  if (nstages > 1) dma(1, 1);
  auto iter = [&](int64_t st, auto bufc) {
    constexpr int B = decltype(bufc)::value;
    // this wave's loads of stage st are in LDS (those of st + 1 may still be
    // in flight), then the barrier.  Not __syncthreads(): its fence would
    // also wait for the next stage's loads.  LDS needs no cache maintenance
    // between waves; the memory clobber keeps LDS accesses on their side.
    if (st + 1 < nstages) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (st + 2 < nstages) dma((B + 2) % kMxStages, st + 2);
    compute(B, 0);
    if (2 * st + 1 < ksteps) compute(B, 1);
  };
  int64_t s = 0;
  do {
    iter(s, MxConst<0>{});
    if (s + 1 >= nstages) break;
    iter(s + 1, MxConst<1>{});
    if (s + 2 >= nstages) break;
    iter(s + 2, MxConst<2>{});
    s += 3;
  } while (s < nstages);
  mfma_drain();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc_fence(acc[i][j]);

  // lane l of tile (i, j): rows 16i + 4q + r, column 16j + l%16
  const int64_t m0 = mt0 + wm * 64, n0 = nt0 + wn * 64;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + 16 * j + fr;
    if (n >= N) continue;
    const float bv = bias ? f16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 16 * i + 4 * q + r;
        if (m >= M) continue;
        const float v = acc[i][j][r] + bv;
        if constexpr (ODT == kF32)
          reinterpret_cast<float *>(y)[m * N + n] = v;
        else if constexpr (ODT == kF16)
          reinterpret_cast<uint16_t *>(y)[m * N + n] = f32_to_f16_bits(v);
        else
          reinterpret_cast<uint16_t *>(y)[m * N + n] = f32_to_bf16_bits(v);
      }
  }
}

template <int DT>
static void launch_mxq(dim3 grid, hipStream_t st, const void *src, int64_t rows, int64_t I, const int16_t *pairs,
                       const float *theta, const float *cs, int krot, int gm, uint8_t *codes, uint8_t *scales) {
  hipLaunchKernelGGL((mx_quant_kernel<DT, true>), grid, dim3(256), 0, st, src, rows, I, pairs, theta, cs, krot, gm,
                     codes, scales);
}

hipError_t launch_mx_quantize_weight(const void *w, int dt, int64_t rows, int64_t I, const int16_t *pairs,
                                     const float *theta, const float *cs, int krot, int group, uint8_t *codes,
                                     uint8_t *scales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)(I / kG), (unsigned)((rows + 63) / 64));
  const int gm = kG - group;
  if (dt == kF16) launch_mxq<kF16>(grid, st, w, rows, I, pairs, theta, cs, krot, gm, codes, scales);
  else if (dt == kBF16) launch_mxq<kBF16>(grid, st, w, rows, I, pairs, theta, cs, krot, gm, codes, scales);
  else launch_mxq<kF32>(grid, st, w, rows, I, pairs, theta, cs, krot, gm, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t *ac, const uint8_t *as, int64_t M, const uint8_t *wc, const uint8_t *ws,
                          int64_t N, int64_t K, const uint16_t *bias, void *y, int y_dt, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)(((M + kMxBM - 1) / kMxBM) * ((N + kMxBN - 1) / kMxBN)));
  if (y_dt == kF32)
    hipLaunchKernelGGL((mx_gemm_kernel<kF32>), grid, dim3(512), 0, st, ac, as, M, wc, ws, N, K, bias, y);
  else if (y_dt == kF16)
    hipLaunchKernelGGL((mx_gemm_kernel<kF16>), grid, dim3(512), 0, st, ac, as, M, wc, ws, N, K, bias, y);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<kBF16>), grid, dim3(512), 0, st, ac, as, M, wc, ws, N, K, bias, y);
  return hipGetLastError();
}

}  // namespace paro

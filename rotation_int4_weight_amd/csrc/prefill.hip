// prefill.hip - many-token rotated W4A16 linear: MFMA GEMM over the rotated
// activations, with each packed weight tile dequantized once into LDS.
//
//   y[m][n] = sum_k x_r[m][k] * w[k][n] + b[n],   w[k][n] = (q[k][n] - z[g][n]) * s[g][n]
//
// ("ParoQuant" wiki, Activation and weight transforms: Y = X_r Q(W_r)^T + b;
// Triton plans and tuning: unpack the 4-bit tile, subtract zero points,
// multiply by group scales, accumulate in fp32.)
//
// Tiling: a workgroup (4 waves, one per SIMD) computes a BM=256 x BN=128 tile
// of y; wave w owns rows 64w..64w+63 (4 MFMA row tiles) and all 128 columns
// (8 column tiles): 32 v_mfma_f32_16x16x32 per 32-deep k step.
//   * A (rotated activations, [tokens][I]) is read straight into MFMA
//     fragments (lane l: row l&15, 8 consecutive k of block l>>4) with buffer
//     loads two k steps ahead.  The buffer descriptor's base moves along k in
//     scalar registers, and its record count ends at the last token, so rows
//     past the end read as zeros without any per-lane test.  The k loop is
//     unrolled by a whole 128-row group, so every prefetch buffer is consumed
//     in place (no register copies of load targets).
//   * B: each k step the workgroup turns its 32 x 128 packed tile (512 words:
//     each thread one word of two adjacent rows) into compute-dtype weights in
//     a double-buffered LDS tile [column][k].  fp16: a byte permute and an OR
//     with 0x6400 make 1024+q exactly, then one packed add of -(1024+z) and one
//     packed multiply by s give (q-z)*s rounded once, two weights per
//     instruction.  bf16 (no packed bf16 arithmetic): byte-to-float converts,
//     an fma q*s + (-z*s) that is exact in fp32, and a paired round to bf16.
//     Zero points and scales are decoded once per group.  Waves read B
//     fragments as two 8-byte LDS loads; the column stride of 36 halves keeps
//     those reads free of bank conflicts.
#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kBM = 256, kBN = 128, kBK = 32;
constexpr int kStepsPerGroup = kG / kBK;
constexpr int kBStride = kBK + 4;  // halves per LDS column (72 bytes)
// Buffer descriptor word 3 for raw (untyped) buffers on the gfx9 family.
constexpr int kRawBufferWord3 = 0x00020000;

template <int DT>
__device__ __forceinline__ f32x4 mfma_tile(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// Per-group constants of one expansion thread, for the 8 nibble slots of its
// word (slot s = column 8w + awq_col(s)).  fp16: packed pairs -(1024+z) and
// (s, s); bf16: -z*s and s in fp32.
template <int DT>
struct GroupConsts;
template <>
struct GroupConsts<kF16> {
  f16x2 zo[8], sc[8];
  __device__ __forceinline__ void decode(u32x4 sw, uint32_t zw) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = awq_col(s);
      const uint32_t h = (sw[c >> 1] >> (16 * (c & 1))) & 0xffffu;
      const uint32_t z = 0xe400u | ((zw >> (4 * s)) & 0xfu);  // fp16 bits of -(1024 + z)
      sc[s] = __builtin_bit_cast(f16x2, h | (h << 16));
      zo[s] = __builtin_bit_cast(f16x2, z | (z << 16));
    }
  }
};
template <>
struct GroupConsts<kBF16> {
  float zs[8], sc[8];
  __device__ __forceinline__ void decode(u32x4 sw, uint32_t zw) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = awq_col(s);
      sc[s] = f16_bits_to_f32((sw[c >> 1] >> (16 * (c & 1))) & 0xffffu);
      zs[s] = -(float)((zw >> (4 * s)) & 0xfu) * sc[s];  // exact: 4-bit x 11-bit
    }
  }
};

// Dequantize one packed word of rows 2rp (ra) and 2rp+1 (rb) into the LDS
// tile: slot s goes to column 8w + awq_col(s), k = 2rp, 2rp+1 as one u32.
template <int DT>
__device__ __forceinline__ void expand_pair_to_lds(uint32_t ra, uint32_t rb, const GroupConsts<DT> &gc,
                                                   uint16_t *bl, int w, int rp) {
  uint32_t v[8];
  if constexpr (DT == kF16) {
    // P = [ra.b0, ra.b2, rb.b0, rb.b2], Q = [ra.b1, ra.b3, rb.b1, rb.b3]: after
    // the shifts below, bits 0..3 and 16..19 hold slot s of ra and of rb.
    const uint32_t P = __builtin_amdgcn_perm(ra, rb, 0x02000604u);
    const uint32_t Q = __builtin_amdgcn_perm(ra, rb, 0x03010705u);
    const uint32_t M = 0x000f000fu, E = 0x64006400u;
    const uint32_t e[8] = {(P & M) | E,         ((P >> 4) & M) | E, (Q & M) | E,         ((Q >> 4) & M) | E,
                           ((P >> 8) & M) | E, ((P >> 12) & M) | E, ((Q >> 8) & M) | E, ((Q >> 12) & M) | E};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      f16x2 h = __builtin_bit_cast(f16x2, e[s]) + gc.zo[s];  // q - z, exact
      h = h * gc.sc[s];                                      // one rounding
      v[s] = __builtin_bit_cast(uint32_t, h);
    }
  } else {
    // bytes of lo_* hold slots 0,2,4,6 and of hi_* slots 1,3,5,7.  The empty
    // asm hides the masks from the optimizer, which would otherwise merge
    // them into per-nibble bit-field extracts instead of using the
    // byte-to-float converts (v_cvt_f32_ubyte0..3).
    uint32_t lo_a = ra & 0x0f0f0f0fu, hi_a = (ra >> 4) & 0x0f0f0f0fu;
    uint32_t lo_b = rb & 0x0f0f0f0fu, hi_b = (rb >> 4) & 0x0f0f0f0fu;
    asm volatile("" : "+v"(lo_a), "+v"(hi_a), "+v"(lo_b), "+v"(hi_b));
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t wa = (s & 1) ? hi_a : lo_a, wb = (s & 1) ? hi_b : lo_b;
      const int sh = 8 * (s >> 1);
      const float qa = (float)((wa >> sh) & 0xffu), qb = (float)((wb >> sh) & 0xffu);
      const f32x2 d = {__builtin_fmaf(qa, gc.sc[s], gc.zs[s]), __builtin_fmaf(qb, gc.sc[s], gc.zs[s])};
      v[s] = __builtin_bit_cast(uint32_t, __builtin_convertvector(d, bf16x2));  // one paired RNE
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
    *reinterpret_cast<uint32_t *>(bl + (8 * w + awq_col(s)) * kBStride + 2 * rp) = v[s];
}

template <int DT>
__global__ void __launch_bounds__(256)
prefill_gemm_kernel(LinearArgs a, const uint16_t *__restrict__ xr) {
  __shared__ __attribute__((aligned(16))) uint16_t bl[2][kBN * kBStride];
  const int lane = lane_id(), wave = wave_id();
  const int64_t I = a.I, O = a.O, W = O / 8, M = a.tokens;
  // XCD-local order: consecutive logical tiles (the N tiles of one M block)
  // share an XCD and its L2.
  const int n_tiles = (int)((O + kBN - 1) / kBN), m_tiles = (int)((M + kBM - 1) / kBM);
  const int lwg = xcd_local_order((int)blockIdx.x, n_tiles * m_tiles);
  const int64_t n0 = (int64_t)(lwg % n_tiles) * kBN;
  const int64_t mb = (int64_t)(lwg / n_tiles) * kBM;
  const int nsteps = (int)(I / kBK), ngroups = (int)(I / kG);

  // expansion role: word dw of the tile's 16, rows 2*drp and 2*drp+1 of a step
  const int drp = threadIdx.x & 15, dw = threadIdx.x >> 4;
  const int64_t dword = n0 / 8 + dw;
  const uint32_t dwc = (uint32_t)(dword < W ? dword : W - 1);  // tail tile: any in-bounds word
  const uint32_t w_off = (uint32_t)((2 * drp) * W + dwc) * 4u;
  const uint32_t w_step_bytes = (uint32_t)(kBK * W * 4);

  // fragment role: row fr of a row tile, k block fk
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  // A rows of this workgroup: [mb, mb + rows); the descriptor covers exactly
  // those rows, so fragment rows at or past `rows` load zeros.
  const int64_t rows = (M - mb) < kBM ? (M - mb) : kBM;
  const uint32_t a_bytes = (uint32_t)(rows * I * 2);
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_off[i] = (uint32_t)(((wave * 64 + i * 16 + fr) * I + fk) * 2);
  const char *a_base = reinterpret_cast<const char *>(xr + mb * I);

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](int step, u32x4 af[4]) {
    const int st = step < nsteps ? step : nsteps - 1;  // past the end: any in-bounds step, unused
    const uint32_t kb = (uint32_t)st * (kBK * 2);
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(a_base + kb, a_bytes - kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = __builtin_amdgcn_raw_buffer_load_b128(r, a_off[i], 0, 0);
  };
  struct Words {
    uint32_t ra, rb;
  };
  auto load_words = [&](int step, Words &wd) {
    const int st = step < nsteps ? step : nsteps - 1;
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(a.qweight + (int64_t)st * kBK * W, w_step_bytes);
    wd.ra = __builtin_amdgcn_raw_buffer_load_b32(r, w_off, 0, 0);
    wd.rb = __builtin_amdgcn_raw_buffer_load_b32(r, w_off + (uint32_t)(W * 4), 0, 0);
  };
  struct GroupRaw {
    u32x4 sw;
    uint32_t zw;
  };
  auto load_group = [&](int g, GroupRaw &gr) {
    const int gg = g < ngroups ? g : ngroups - 1;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.scales + (int64_t)gg * O, (uint32_t)(O * 2));
    gr.sw = __builtin_amdgcn_raw_buffer_load_b128(rs, dwc * 16u, 0, 0);
    const __amdgpu_buffer_rsrc_t rz = raw_rsrc(a.qzeros + (int64_t)gg * W, (uint32_t)(W * 4));
    gr.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, dwc * 4u, 0, 0);
  };

  GroupConsts<DT> gc;
  GroupRaw graw;
  Words wd[2];
  u32x4 ab[2][4];
  load_group(0, graw);
  load_words(0, wd[0]);
  load_words(1, wd[1]);
  load_a(0, ab[0]);
  load_a(1, ab[1]);
  gc.decode(graw.sw, graw.zw);
  expand_pair_to_lds<DT>(wd[0].ra, wd[0].rb, gc, bl[0], dw, drp);
  load_words(2, wd[0]);
  __syncthreads();

  // Step s: MFMAs on A[s&1] and LDS tile s&1; refill A[s&1] <- s+2; expand
  // the words of step s+1 into the other tile; refill those words <- s+3;
  // barrier.  The group's next scales/zeros are fetched at its first step
  // and decoded just before the first expansion that needs them.
  auto do_step = [&](int step, u32x4(&A)[4], Words &wnext, const uint16_t *bcur, uint16_t *bnext, bool last_of_group) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(bcur + (j * 16 + fr) * kBStride + fk);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(bcur + (j * 16 + fr) * kBStride + fk + 4);
      const u32x4 bfrag = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma_tile<DT>(A[i], bfrag, acc[i][j]);
    }
    load_a(step + 2, A);
    if (step + 1 < nsteps) {
      if (last_of_group) gc.decode(graw.sw, graw.zw);
      expand_pair_to_lds<DT>(wnext.ra, wnext.rb, gc, bnext, dw, drp);
    }
    load_words(step + 3, wnext);
    __syncthreads();
  };
  for (int g = 0; g < ngroups; ++g) {
    const int s0 = g * kStepsPerGroup;
    load_group(g + 1, graw);
    do_step(s0 + 0, ab[0], wd[1], bl[0], bl[1], false);
    do_step(s0 + 1, ab[1], wd[0], bl[1], bl[0], false);
    do_step(s0 + 2, ab[0], wd[1], bl[0], bl[1], false);
    do_step(s0 + 3, ab[1], wd[0], bl[1], bl[0], true);
  }

  // epilogue: bias in fp32, one rounding to the output dtype
  const int64_t m0 = mb + wave * 64;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t n = n0 + j * 16 + fr;
    if (n >= O) continue;
    const float bias = a.bias ? f16_bits_to_f32(a.bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= M) continue;
        const float v = acc[i][j][r] + bias;
        if (a.y_dt == kF32) reinterpret_cast<float *>(a.y)[row * O + n] = v;
        else if (a.y_dt == kF16) reinterpret_cast<uint16_t *>(a.y)[row * O + n] = f32_to_f16_bits(v);
        else reinterpret_cast<uint16_t *>(a.y)[row * O + n] = f32_to_bf16_bits(v);
      }
    }
  }
}

hipError_t launch_prefill_gemm(const LinearArgs &a, const void *xr, hipStream_t st) {
  dim3 grid((unsigned)(((a.O + kBN - 1) / kBN) * ((a.tokens + kBM - 1) / kBM)));
  const uint16_t *x = reinterpret_cast<const uint16_t *>(xr);
  if (a.x_dt == kF16)
    hipLaunchKernelGGL((prefill_gemm_kernel<kF16>), grid, dim3(256), 0, st, a, x);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<kBF16>), grid, dim3(256), 0, st, a, x);
  return hipGetLastError();
}

}  // namespace paro

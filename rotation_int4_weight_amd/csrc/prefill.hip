// prefill.hip - many-token rotated W4A16 linear: MFMA GEMM over the rotated
// activations, with the packed weight tile dequantized into LDS.
//
//   y[m][n] = sum_k x_r[m][k] * ((q[k][n] - z[k/128][n]) * s[k/128][n]) + b[n]
//
// ("ParoQuant" wiki, Activation and weight transforms: Y = X_r Q(W_r)^T + b;
// Triton plans and tuning: unpack the 4-bit tile, subtract zero points,
// multiply by group scales, accumulate in fp32.)
//
// Tiling: a workgroup (4 waves) computes a BM=256 x BN=128 tile of y; wave w
// owns rows 64w..64w+63 (4 MFMA row tiles) and all 128 columns (8 column
// tiles) and accumulates 32 v_mfma_f32_16x16x32 tiles per 32-deep k step.
//   * A (rotated activations, [tokens][I]) is read straight from global into
//     MFMA fragments (lane l: row l&15, 8 consecutive k of block l>>4),
//     prefetched two k steps ahead.
//   * B: each k step the workgroup expands its 32 x 128 packed tile (512
//     words, two per thread) into a double-buffered LDS tile held as
//     [column][k] in the activation dtype, with the weight value
//     (q - z) * s rounded once to nearest even; waves then read B fragments
//     as two 8-byte LDS loads.  The column stride of 36 halves makes those
//     reads conflict-free (16 lanes of a phase cover all 32 banks) and keeps
//     the dequant stores at two lanes per bank; a thread expands one word of
//     one row pair, and a wave spans all 16 row pairs of 4 words.  fp16: the nibble becomes 1024+q by an OR
//     with 0x6400, then packed fp16 ops subtract 1024+z (exact) and multiply
//     by s; bf16: the nibble is converted to fp32, (q - z) * s is one exact
//     FMA (q*s and z*s are exact in fp32) and the pair is rounded to bf16.
#include "common.hpp"
#include "launch.hpp"

namespace paro {

constexpr int kBM = 256, kBN = 128, kBK = 32;
constexpr int kBStride = kBK + 4;  // halves per LDS column (72 bytes)

template <int DT>
__device__ __forceinline__ f32x4 mfma_tile(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// Dequantize rows (ra: row 2rp, rb: row 2rp+1) of one packed column word into
// eight (k, k+1) pairs, one per column 8w + awq_col(s), and store them at
// B[col][2rp] in LDS.
template <int DT>
__device__ __forceinline__ void dequant_pair_to_lds(uint32_t ra, uint32_t rb, u32x4 sv, uint32_t zw,
                                                    uint16_t *bl, int w, int rp) {
  if constexpr (DT == kF16) {
    const uint32_t P = __builtin_amdgcn_perm(ra, rb, 0x02000604u);  // [ra.b0, ra.b2, rb.b0, rb.b2]
    const uint32_t Q = __builtin_amdgcn_perm(ra, rb, 0x03010705u);  // [ra.b1, ra.b3, rb.b1, rb.b3]
    uint32_t v[8];
    v[0] = P;
    v[1] = P >> 4;
    v[4] = P >> 8;
    v[5] = P >> 12;
    v[2] = Q;
    v[3] = Q >> 4;
    v[6] = Q >> 8;
    v[7] = Q >> 12;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int col = awq_col(s);
      const uint32_t z = (zw >> (4 * s)) & 0xfu;
      const uint32_t sb = (sv[col >> 1] >> (16 * (col & 1))) & 0xffffu;
      const f16x2 qq = __builtin_bit_cast(f16x2, (v[s] & 0x000f000fu) | 0x64006400u);  // 1024 + q
      const _Float16 zz = -__builtin_bit_cast(_Float16, (uint16_t)(0x6400u | z));      // -(1024 + z)
      const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)sb);
      const f16x2 d = (qq + f16x2{zz, zz}) * f16x2{sc, sc};
      *reinterpret_cast<uint32_t *>(bl + (8 * w + col) * kBStride + 2 * rp) = __builtin_bit_cast(uint32_t, d);
    }
  } else {
    const uint32_t a0 = ra & 0x0f0f0f0fu, a1 = (ra >> 4) & 0x0f0f0f0fu;  // slots 0,2,4,6 / 1,3,5,7
    const uint32_t b0 = rb & 0x0f0f0f0fu, b1 = (rb >> 4) & 0x0f0f0f0fu;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int col = awq_col(s);
      const uint32_t z = (zw >> (4 * s)) & 0xfu;
      const float sc = f16_bits_to_f32((sv[col >> 1] >> (16 * (col & 1))) & 0xffffu);
      const float nzs = -(float)z * sc;  // exact: 4-bit times 11-bit significand
      const uint32_t srcA = (s & 1) ? a1 : a0, srcB = (s & 1) ? b1 : b0;
      const int byte = s >> 1;
      const float qa = (float)((srcA >> (8 * byte)) & 0xffu);
      const float qb = (float)((srcB >> (8 * byte)) & 0xffu);
      const float wa = __builtin_fmaf(qa, sc, nzs), wb = __builtin_fmaf(qb, sc, nzs);
      *reinterpret_cast<uint32_t *>(bl + (8 * w + col) * kBStride + 2 * rp) = pack2<kBF16>(wa, wb);
    }
  }
}

template <int DT>
__global__ void __launch_bounds__(256)
prefill_gemm_kernel(LinearArgs a, const uint16_t *__restrict__ xr) {
  __shared__ __attribute__((aligned(16))) uint16_t bl[2][kBN * kBStride];
  const int lane = lane_id(), wave = wave_id();
  const int64_t I = a.I, O = a.O, W = O / 8, M = a.tokens;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * kBM + wave * 64;
  const int nsteps = (int)(I / kBK);

  // dequant role: word dw of the tile, rows 2*drp and 2*drp+1 of each k step
  const int drp = threadIdx.x & 15, dw = threadIdx.x >> 4;
  const int64_t dword = n0 / 8 + dw;
  const bool dvalid = dword < W;

  // fragment role
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_words = [&](int step, uint32_t &ra, uint32_t &rb, u32x4 &sv, uint32_t &zw) {
    if (dvalid && step < nsteps) {
      const int64_t k = (int64_t)step * kBK + 2 * drp;
      const int64_t g = ((int64_t)step * kBK) / kG;
      ra = (uint32_t)a.qweight[k * W + dword];
      rb = (uint32_t)a.qweight[(k + 1) * W + dword];
      sv = *reinterpret_cast<const u32x4 *>(a.scales + g * O + 8 * dword);
      zw = (uint32_t)a.qzeros[g * W + dword];
    } else {
      ra = rb = zw = 0u;
      sv = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_a = [&](int step, u32x4 af[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + i * 16 + fr;
      if (row < M && step < nsteps)
        af[i] = *reinterpret_cast<const u32x4 *>(xr + row * I + (int64_t)step * kBK + fk);
      else
        af[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // prologue: B tile of step 0 into LDS buffer 0; words of step 1 and A of
  // steps 0 and 1 in registers
  uint32_t ra, rb, zw;
  u32x4 sv;
  load_words(0, ra, rb, sv, zw);
  dequant_pair_to_lds<DT>(ra, rb, sv, zw, bl[0], dw, drp);
  load_words(1, ra, rb, sv, zw);
  u32x4 a_cur[4], a_nxt[4];
  load_a(0, a_cur);
  load_a(1, a_nxt);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    // expand the next step's tile into the other buffer, fetch the one after
    if (step + 1 < nsteps) dequant_pair_to_lds<DT>(ra, rb, sv, zw, bl[buf ^ 1], dw, drp);
    load_words(step + 2, ra, rb, sv, zw);

    const uint16_t *bb = bl[buf];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(bb + (j * 16 + fr) * kBStride + fk);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(bb + (j * 16 + fr) * kBStride + fk + 4);
      const u32x4 bfrag = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma_tile<DT>(a_cur[i], bfrag, acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a_cur[i] = a_nxt[i];
    load_a(step + 2, a_nxt);
    __syncthreads();
  }

  // epilogue: bias in fp32, one rounding to the output dtype
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
  dim3 grid((unsigned)((a.O + kBN - 1) / kBN), (unsigned)((a.tokens + kBM - 1) / kBM));
  const uint16_t *x = reinterpret_cast<const uint16_t *>(xr);
  if (a.x_dt == kF16)
    hipLaunchKernelGGL((prefill_gemm_kernel<kF16>), grid, dim3(256), 0, st, a, x);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<kBF16>), grid, dim3(256), 0, st, a, x);
  return hipGetLastError();
}

}  // namespace paro

// unpack_dequant.hip - AWQ nibble unpack and affine dequantization.
//
// "ParoQuant" wiki, Stored tensors: qweight (I, O/8) and qzeros (I/G, O/8),
// eight 4-bit values per int32 word; Triton plans and tuning: subtract the
// zero points, multiply by the group scales.  "GPTQ, GPTAQ, and RTN" wiki,
// quantizer: x_hat = scale * (q - zero).
//
// One thread per packed word (row k, word w): it extracts the 8 codes with
// logical shifts, writes them in column order, and writes (q - z) * s, which
// is exact in fp32 (|q - z| <= 15 times an 11-bit fp16 significand) and then
// rounded once to nearest even into the output dtype.
#include "common.hpp"
#include "launch.hpp"

namespace paro {

template <int WDT>
__global__ void __launch_bounds__(256)
unpack_dequant_kernel(const int32_t *__restrict__ qweight, const int32_t *__restrict__ qzeros,
                      const uint16_t *__restrict__ scales, int64_t I, int64_t O, int64_t G,
                      uint8_t *__restrict__ q_out, uint8_t *__restrict__ z_out, void *__restrict__ w_out) {
  const int64_t W = O / 8;
  const int64_t total = I * W;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = e / W, w = e - k * W, g = k / G;
    const uint32_t qw = (uint32_t)qweight[e];
    const uint32_t zw = (uint32_t)qzeros[g * W + w];
    int q[8], z[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      q[awq_col(s)] = (int)((qw >> (4 * s)) & 0xfu);
      z[awq_col(s)] = (int)((zw >> (4 * s)) & 0xfu);
    }
    if (q_out) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo |= (uint32_t)q[c] << (8 * c);
        hi |= (uint32_t)q[c + 4] << (8 * c);
      }
      *reinterpret_cast<u32x2 *>(q_out + k * O + 8 * w) = u32x2{lo, hi};
    }
    if (z_out && (k % G) == 0) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo |= (uint32_t)z[c] << (8 * c);
        hi |= (uint32_t)z[c + 4] << (8 * c);
      }
      *reinterpret_cast<u32x2 *>(z_out + g * O + 8 * w) = u32x2{lo, hi};
    }
    if (w_out) {
      const u32x4 sv = *reinterpret_cast<const u32x4 *>(scales + g * O + 8 * w);
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sb = (sv[c >> 1] >> (16 * (c & 1))) & 0xffffu;
        v[c] = (float)(q[c] - z[c]) * f16_bits_to_f32(sb);
      }
      if constexpr (WDT == kF32) {
        float *o = reinterpret_cast<float *>(w_out) + k * O + 8 * w;
        *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        u32x4 pk;
#pragma unroll
        for (int c = 0; c < 4; ++c) pk[c] = pack2<WDT>(v[2 * c], v[2 * c + 1]);
        *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(w_out) + k * O + 8 * w) = pk;
      }
    }
  }
}

hipError_t launch_unpack_dequant(const int32_t *qweight, const int32_t *qzeros, const uint16_t *scales,
                                 int64_t I, int64_t O, int64_t G, uint8_t *q_out, uint8_t *z_out,
                                 void *w_out, int w_dt, hipStream_t st) {
  const int64_t total = I * (O / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  dim3 grid((unsigned)blocks);
  if (w_dt == kF16)
    hipLaunchKernelGGL((unpack_dequant_kernel<kF16>), grid, dim3(256), 0, st, qweight, qzeros, scales, I, O,
                       G, q_out, z_out, w_out);
  else if (w_dt == kBF16)
    hipLaunchKernelGGL((unpack_dequant_kernel<kBF16>), grid, dim3(256), 0, st, qweight, qzeros, scales, I, O,
                       G, q_out, z_out, w_out);
  else
    hipLaunchKernelGGL((unpack_dequant_kernel<kF32>), grid, dim3(256), 0, st, qweight, qzeros, scales, I, O,
                       G, q_out, z_out, w_out);
  return hipGetLastError();
}

}  // namespace paro

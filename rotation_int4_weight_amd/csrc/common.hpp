// common.hpp - device helpers shared by the libparo kernels (gfx950 / CDNA4).
//
// Formats: fp16 = IEEE binary16, bf16 = upper half of binary32.  Every
// narrowing is round-to-nearest-even (the hardware default mode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace paro {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// dtype codes of the C-ABI (paro_dtype)
enum : int { kF16 = 0, kBF16 = 1, kF32 = 2 };

// Group width of the GPU path and its pair count.
constexpr int kG = 128;
constexpr int kPairs = kG / 2;

// AWQ word layout: bits 4s..4s+3 of a packed word hold column 8w + awq_col(s);
// the interleave puts the even columns 0,2,4,6 in slots 0..3 and the odd
// columns 1,3,5,7 in slots 4..7.
__host__ __device__ constexpr int awq_col(int slot) { return ((slot & 3) << 1) | (slot >> 2); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}
template <int DT>
__device__ __forceinline__ float act_to_f32(uint32_t bits16) {
  if constexpr (DT == kF16) return f16_bits_to_f32(bits16);
  else return bf16_bits_to_f32(bits16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
// Two floats -> packed pair (lo in bits 0..15), RNE.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == kF16) {
    return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
  } else {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
  }
}

// Wavefront-scope ordering of LDS traffic between lanes of one wave: LDS
// operations of a wave execute in issue order, so only the compiler needs to
// be kept from reordering across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Workgroups of a launch are handed to the 8 XCDs round-robin by id.  This
// maps launch id b to a logical index so that each XCD receives a contiguous
// run of logical indices (a bijection on [0, total); ids past the last full
// round keep their own index).  Only data placement in the XCDs' L2 caches
// depends on it, never correctness.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_local_order(int b, int total) {
  const int q = total / kXcds;
  if (b >= q * kXcds) return b;
  return (b % kXcds) * q + b / kXcds;
}
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// Pairwise Givens rotation of NR token rows of one 128-channel group.
//
// The rows live in LDS as fp32, row r at xs[r * rs + c] (c < 128).  Lane p of
// the calling wave owns pair p at every stage: it reads the pair's two
// channels for all NR rows, applies
//     a' =  a cos(theta) + b sin(theta),   b' = -a sin(theta) + b cos(theta)
// and writes them back.  Pairs of a stage are disjoint, so no lane touches
// another's channels within a stage; stages are ordered by wave_lds_sync().
// NR is a compile-time row count (callers pad with zero rows), so the row
// loops are branch-free and every load of a stage is issued before its first
// use.
//   pairs_g : &pairs[0][g*128]   (row stride `pstride` int16 = I)
//   theta_g : &theta[0][g*64]    (row stride `tstride` floats = I/2)
// Pair indices are masked into the group, so a bad schedule cannot read or
// write outside the group's 128 channels.
//
// Rotation groups of G = 32 or 64 channels: pairs never leave their group,
// so a 128-channel block holds 128/G groups and is rotated as one block.  The
// stored pair indices are local to their G-group; lane p's pair (word slots
// 2p, 2p+1) lies in group (2p)/G of the block, so its block-local indices
// are the stored ones plus (2p) & (128 - G).  gmask = 128 - G (0 for 128).
//
// The pair words and angles of the first kStageRegs stages can be loaded
// early (RotParams::load), long before the rows are rotated, so that their
// latency hides behind other memory traffic; later stages, if any, are
// fetched as they are applied.
// ---------------------------------------------------------------------------
constexpr int kStageRegs = 8;

__device__ __forceinline__ uint32_t block_pair_word(uint32_t w, int lane, int gmask) {
  return w + (uint32_t)((2 * lane) & gmask) * 0x00010001u;
}
__device__ __forceinline__ uint32_t load_pair_word(const int16_t *__restrict__ pairs_g, int64_t pstride, int t,
                                                   int lane, int gmask) {
  return block_pair_word(*reinterpret_cast<const uint32_t *>(pairs_g + (int64_t)t * pstride + 2 * lane), lane,
                         gmask);
}

struct RotParams {
  uint32_t pw[kStageRegs];
  float th[kStageRegs];
  __device__ __forceinline__ void load(const int16_t *__restrict__ pairs_g, int64_t pstride,
                                       const float *__restrict__ theta_g, int64_t tstride, int krot,
                                       int lane, int gmask) {
#pragma unroll
    for (int u = 0; u < kStageRegs; ++u) {
      const int t = u < krot ? u : 0;  // stages past krot are never applied
      pw[u] = load_pair_word(pairs_g, pstride, t, lane, gmask);
      th[u] = theta_g[(int64_t)t * tstride + lane];
    }
  }
};

template <int NR>
__device__ __forceinline__ void rotate_stage(float *xs, int rs, uint32_t pw, float cs, float sn) {
  const int a = (int)(pw & (kG - 1));
  const int b = (int)((pw >> 16) & (kG - 1));
  float va[NR], vb[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    va[m] = xs[m * rs + a];
    vb[m] = xs[m * rs + b];
  }
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    // explicit contraction: every kernel rounds the stage identically
    xs[m * rs + a] = __builtin_fmaf(va[m], cs, vb[m] * sn);
    xs[m * rs + b] = __builtin_fmaf(vb[m], cs, -(va[m] * sn));
  }
  wave_lds_sync();
}

template <int NR>
__device__ __forceinline__ void rotate_rows_lds(float *xs, int rs, const RotParams &rp,
                                                const int16_t *__restrict__ pairs_g, int64_t pstride,
                                                const float *__restrict__ theta_g, int64_t tstride,
                                                int krot, int lane, int gmask) {
  float cs[kStageRegs], sn[kStageRegs];
#pragma unroll
  for (int u = 0; u < kStageRegs; ++u) __sincosf(rp.th[u], &sn[u], &cs[u]);
#pragma unroll
  for (int u = 0; u < kStageRegs; ++u)
    if (u < krot) rotate_stage<NR>(xs, rs, rp.pw[u], cs[u], sn[u]);
  for (int t = kStageRegs; t < krot; ++t) {
    const uint32_t pw = load_pair_word(pairs_g, pstride, t, lane, gmask);
    float c, s;
    __sincosf(theta_g[(int64_t)t * tstride + lane], &s, &c);
    rotate_stage<NR>(xs, rs, pw, c, s);
  }
}

}  // namespace paro

// mfma.hpp - matrix-core and buffer-load helpers shared by the GEMM-shaped
// kernels (prefill contraction, dense-matrix rotation).
#pragma once

#include "common.hpp"

namespace paro {

// Buffer descriptor word 3 for raw (untyped) buffers on the gfx9 family.
constexpr int kRawBufferWord3 = 0x00020000;

// c += A * B on one 16x16 tile (v_mfma_f32_16x16x32_{f16,bf16}), with c tied
// to one AGPR quadruple.  Written as asm because the builtin lets the
// register allocator pick a destination other than c, and it then shuffles
// accumulators between loop iterations with v_accvgpr moves that each wait
// for the MFMA just issued.  The compiler does not see these as MFMAs, so
// the wait states before the accumulators are read back are inserted by hand
// (mfma_drain); operands come straight from buffer and LDS loads, which need
// none.
template <int DT>
__device__ __forceinline__ void mfma_acc(const u32x4 &a, const u32x4 &b, f32x4 &c) {
  if constexpr (DT == kF16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// mfma_acc for operands that a VALU instruction may have written just before
// the MFMA, e.g. a copy out of an AGPR that the register allocator inserts
// under pressure: the hardware needs wait states between a VALU write of a
// VGPR and an MFMA reading it, and the compiler inserts none before asm.
template <int DT>
__device__ __forceinline__ void mfma_acc_after_valu(const u32x4 &a, const u32x4 &b, f32x4 &c) {
  if constexpr (DT == kF16)
    asm volatile("s_nop 2\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 2\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// D = A * B + c on one 16x16 tile through the builtin (the compiler tracks
// its latency); for short-lived products whose result a VALU reads next.
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, f32x4 c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
// 64 wait states: more than any MFMA needs before a VALU reads its result.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15");
  __builtin_amdgcn_sched_barrier(0);
}

// Ties c to an (empty) volatile asm placed after mfma_drain, so that the
// compiler cannot move the reads of c above the drain.
__device__ __forceinline__ void acc_fence(f32x4 &c) { asm volatile("" : "+a"(c)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferWord3);
}

}  // namespace paro

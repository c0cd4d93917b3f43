// launch.hpp - internal host launchers of the libparo kernels.
//
// The C-ABI layer (paro_abi.cpp) validates every argument before calling
// these; they only compute grids and enqueue kernels on `st`, returning the
// launch status.  All pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paro.h"

namespace paro {

// `group`: the rotation / quantization group size G (32, 64 or 128); the
// kernels rotate 128-channel blocks with the pair indices rebased into the
// block (block_pair_word in common.hpp).
hipError_t launch_scale_rotate(const uint16_t *x, int x_dt, void *xr, int xr_dt, int64_t tokens, int64_t I,
                               const int16_t *pairs, const float *theta, const float *cs, int krot, int group,
                               hipStream_t st);

// One rotation group over the whole row (G = I): scaled rows staged in LDS
// (full_row_rows(I) rows per workgroup, R * I * 4 <= kFullRowLdsBytes), the
// stages applied across the workgroup.  tiled: output in the prefill GEMM's
// tiled layout (activation dtype, pad rows zero); else row-major in xr_dt.
constexpr int64_t kFullRowLdsBytes = 65536;
constexpr int64_t kMaxFullRowDim = kFullRowLdsBytes / 4;  // I <= 16384
int full_row_rows(int64_t I);
hipError_t launch_scale_rotate_full(const uint16_t *x, int x_dt, void *xr, int xr_dt, bool tiled, int64_t tokens,
                                    int64_t I, const int16_t *pairs, const float *theta, const float *cs, int krot,
                                    hipStream_t st);

hipError_t launch_unpack_dequant(const int32_t *qweight, const int32_t *qzeros, const uint16_t *scales,
                                 int64_t I, int64_t O, int64_t G, uint8_t *q_out, uint8_t *z_out,
                                 void *w_out, int w_dt, hipStream_t st);

// Everything one linear launch needs (device pointers; sizes already checked).
struct LinearArgs {
  int64_t I, O, tokens;
  int krot;
  int group;  // G: 32, 64 or 128 (rotation pairs and quantization groups), or I (one group per row)
  // MoE (prefill only): experts > 0 stacked experts sharing the rotation,
  // rows of expert e in [expert_offsets[e], expert_offsets[e+1]) (device)
  int experts;
  const int64_t *expert_offsets;
  const int16_t *pairs;
  const float *theta;
  const float *cs;
  const int32_t *qweight;
  const int32_t *qzeros;
  const uint16_t *scales;
  const uint16_t *bias;  // may be null
  const void *x;         // [tokens][I] act dtype
  int x_dt;              // kF16 / kBF16
  void *y;               // [tokens][O]
  int y_dt;              // x_dt or kF32
};

// Decode (tokens <= 16): split-K MFMA GEMV.  With `xr` == nullptr the
// rotation runs fused in each workgroup's prologue; otherwise `xr` holds the
// rotated activations ([tokens][I], x dtype) and is read directly.
struct DecodePlan {
  int wpl;        // packed words per lane and row (1 or 2)
  int ksw;        // 32-row k-steps per wave (a workgroup covers nw * ksw)
  int nw;         // waves per workgroup (4 or 8)
  int ntile;      // output columns per workgroup (= 128 * wpl)
  int n_tiles;    // ceil(O / ntile)
  int splits;     // workgroups along K (ceil(I/32 / (nw * ksw)))
};
// group < 128: one k-step per wave, so every k-step folds with its own
// group's scale and zero point.
DecodePlan plan_decode(int64_t I, int64_t O, int64_t tokens, bool fused, int group = 128);
// Bytes of fp32 split-K partial sums the plan needs (0 with one split).
size_t decode_partial_bytes(const DecodePlan &p, int64_t tokens, int64_t O);
// counters: >= n_tiles zeroed uint32 (left zeroed); partials: decode_partial_bytes.
hipError_t launch_decode(const LinearArgs &a, const DecodePlan &p, const void *xr, uint32_t *counters,
                         float *partials, hipStream_t st);

// Fragment-major tiled layout of rotated activations for the prefill GEMM
// (x dtype).  Rows are padded to a multiple of 16 with zeros.  Each 16-row x
// 32-column block is 1 KB, contiguous, in the order one
// v_mfma_f32_16x16x32 A operand is held across the 64 lanes:
//   element (m, k) at half index
//     ((m/16) * (I/32) + k/32) * 512 + (((k%32)/8) * 16 + m%16) * 8 + k%8
// so one 16-byte load per lane fetches a whole fragment from 8 full cache
// lines.  Size: tiled_rows(tokens) * I * 2 bytes.
__host__ __device__ inline int64_t tiled_rows(int64_t tokens) { return (tokens + 15) / 16 * 16; }

// Dense form of the rotation: R'_g = diag(cs_g) . R_g per 128-channel group,
// stored as H + L in the activation dtype (rot_mat_bytes(I) bytes), and
// X_r = X . (H + L) on the matrix cores, written in the tiled layout (pad
// rows zero).
size_t rot_mat_bytes(int64_t I);
hipError_t launch_rot_build(int x_dt, int64_t I, const int16_t *pairs, const float *theta, const float *cs,
                            int krot, int group, uint16_t *hl, hipStream_t st);
hipError_t launch_rot_apply(const uint16_t *x, int x_dt, uint16_t *xt, int64_t tokens, int64_t I,
                            const uint16_t *hl, hipStream_t st);
// The same product with an MXFP4 epilogue: codes [tokens][I/2], scales
// [tokens][I/32] (see mx.hpp) instead of the tiled X_r.
hipError_t launch_rot_apply_mx(const uint16_t *x, int x_dt, int64_t tokens, int64_t I, const uint16_t *hl,
                               uint8_t *codes, uint8_t *scales, hipStream_t st);
// Row-major [tokens][I] (2-byte elements) -> tiled layout (pad rows zero).
hipError_t launch_retile(const uint16_t *xr, uint16_t *xt, int64_t tokens, int64_t I, hipStream_t st);

// Prefill: MFMA GEMM over rotated activations in the tiled layout.
hipError_t launch_prefill_gemm(const LinearArgs &a, const uint16_t *xt, hipStream_t st);
// Several dense layers of one shape (a's I, O, tokens, group, dtypes) in one
// launch: layer i takes its weights, bias and output from the table and its
// rotated activations from xt[i]; the launch covers the union of the
// layers' output tiles.  a's own pointers are not read.
constexpr int kMaxMultiLayers = 4;
struct LayerTable {
  int n;  // layers, 1..kMaxMultiLayers
  const int32_t *qweight[kMaxMultiLayers];
  const int32_t *qzeros[kMaxMultiLayers];
  const uint16_t *scales[kMaxMultiLayers];
  const uint16_t *bias[kMaxMultiLayers];  // entries may be null
  const uint16_t *xt[kMaxMultiLayers];
  void *y[kMaxMultiLayers];
  int64_t o[kMaxMultiLayers];         // out_features of each layer (dense launches)
  int32_t tile0[kMaxMultiLayers + 1];  // first output tile of each layer; tile0[n]: all tiles (set by the launcher)
};
hipError_t launch_prefill_gemm_multi(const LinearArgs &a, const LayerTable &lt, hipStream_t st);
// Upper bound on the (expert, 256-row tile) work items of a MoE call.
int64_t moe_work_tiles(int64_t tokens, int experts);

// W_r = W D R, group quantization and AWQ packing (the offline step):
// w [O][I] (F16, BF16 or F32); qweight [I][O/8], qzeros [I/G][O/8],
// scales [I/G][O] fp16 (G = group).
hipError_t launch_quantize_pack(const void *w, int w_dt, bool sym, int64_t O, int64_t I, const int16_t *pairs,
                                const float *theta, const float *cs, int krot, int group, int32_t *qweight,
                                int32_t *qzeros,
                                uint16_t *scales, hipStream_t st);

// Backward of the scaling and rotation: x [tokens][I] (F16/BF16), g = dL/dx_r
// [tokens][I] (F32 or x's dtype) -> gx [tokens][I] (F32 or x's dtype),
// gtheta [krot][I/2] fp32, gcs [I] fp32, with `partial` as workspace
// (rot_backward_partial_bytes bytes, 256-byte aligned regions inside).
size_t rot_backward_partial_bytes(int64_t tokens, int64_t I, int krot);
hipError_t launch_rot_backward(const void *x, int x_dt, const void *g, int g_dt, int64_t tokens, int64_t I,
                               const int16_t *pairs, const float *theta, const float *cs, int krot, int group,
                               void *gx,
                               int gx_dt, float *gtheta, float *gcs, float *partial, hipStream_t st);

// MXFP4 (32-element E8M0 blocks, E2M1 codes; mx.hpp) of the transformed
// weight rows W . D . R: w [rows][I] -> codes [rows][I/2], scales [rows][I/32].
hipError_t launch_mx_quantize_weight(const void *w, int dt, int64_t rows, int64_t I, const int16_t *pairs,
                                     const float *theta, const float *cs, int krot, int group, uint8_t *codes,
                                     uint8_t *scales, hipStream_t st);
// y [M][N] = A . W^T (+ bias) on the block-scaled FP4 matrix cores.
hipError_t launch_mx_gemm(const uint8_t *ac, const uint8_t *as, int64_t M, const uint8_t *wc, const uint8_t *ws,
                          int64_t N, int64_t K, const uint16_t *bias, void *y, int y_dt, hipStream_t st);

// The allocation-free linear's scratch (noalloc.hip): one device array of
// kNoallocScratchBytes per GPU, held until the process ends.  noalloc_scratch
// returns the address of the stream's device's copy, setting it up on the
// first call on that device (hipGetSymbolAddress with the device current,
// then the first zero_bytes cleared by a fill kernel on `st`); that first call
// must not be made under graph capture (hipErrorStreamCaptureUnsupported).
constexpr size_t kNoallocScratchBytes = PARO_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(hipStream_t st, size_t zero_bytes, void **ptr);

}  // namespace paro

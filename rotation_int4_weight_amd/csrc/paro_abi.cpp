// paro_abi.cpp - C-ABI of libparo: argument validation, path choice,
// workspace layout and launch-error mapping.  Declarations and the contract
// of every entry point are in include/paro.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "launch.hpp"
#include "paro.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PARO_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxTokens = int64_t(1) << 21;  // keeps every grid dimension < 65536
constexpr int kMaxKrot = 64;
// The prefill GEMM addresses a 256-row activation tile with 32-bit buffer
// offsets (256 * I * 2 bytes < 2^32).
constexpr int64_t kMaxDim = int64_t(1) << 22;
constexpr int64_t kMaxOut = int64_t(1) << 21;
// Every workspace starts with a fixed counter area for the split-K
// reduction (one 32-bit counter on its own 128-byte line per 128-column tile,
// at most kMaxOut/128 tiles), so a zero-filled workspace stays valid across
// shapes and paths: no path ever writes anything but zeros-at-exit into it.
constexpr size_t kCounterBytes = (size_t)(kMaxOut / 128) * 128;

int64_t group_of(const paro_w4_layer *L) { return L->group_size == -1 ? L->in_features : L->group_size; }

// Shape rules of the method ("ParoQuant" wiki: even groups dividing I; AWQ
// packing needs O % 8 == 0; krot >= 1).
int check_method_shape(const paro_w4_layer *L) {
  if (!L) return fail(PARO_ERR_NULL, "layer is NULL");
  const int64_t I = L->in_features, O = L->out_features, G = group_of(L);
  if (I <= 0 || O <= 0) return fail(PARO_ERR_SHAPE, "in_features=%lld out_features=%lld must be positive",
                                    (long long)I, (long long)O);
  if (O % 8) return fail(PARO_ERR_SHAPE, "out_features=%lld is not a multiple of 8", (long long)O);
  if (G <= 0 || G % 2 || I % G)
    return fail(PARO_ERR_SHAPE, "group_size=%d must be even and divide in_features=%lld", L->group_size,
                (long long)I);
  if (L->krot < 1) return fail(PARO_ERR_SHAPE, "krot=%d must be >= 1", L->krot);
  return PARO_OK;
}

// One rotation and quantization group over the whole row: group_size -1
// (or G == I) beyond the 128-channel block sizes.
bool full_row(const paro_w4_layer *L) {
  const int64_t G = group_of(L);
  return G == L->in_features && G != 32 && G != 64 && G != 128;
}

// What the GPU kernels support on top of the method's rules.  rows: the
// entry point also takes one group over the whole row (the linear, the
// row-major rotation, the tiled contraction, the unpack).
int check_gpu_shape(const paro_w4_layer *L, bool rows = false) {
  int rc = check_method_shape(L);
  if (rc) return rc;
  const int64_t G = group_of(L);
  if (full_row(L)) {
    if (!rows)
      return fail(PARO_ERR_UNSUPPORTED,
                  "group_size=%d (one group over all %lld channels): this entry point takes 32, 64 and 128; the "
                  "linear, paro_scale_rotate, paro_w4a16_linear_tiled and paro_w4_unpack_dequant take it",
                  L->group_size, (long long)L->in_features);
    if (L->in_features > paro::kMaxFullRowDim)
      return fail(PARO_ERR_UNSUPPORTED, "one group over the row: in_features=%lld exceeds %lld",
                  (long long)L->in_features, (long long)paro::kMaxFullRowDim);
  } else if (G != 32 && G != 64 && G != 128) {
    return fail(PARO_ERR_UNSUPPORTED, "group_size=%d: the GPU path supports 32, 64, 128 and -1 (the whole row)",
                L->group_size);
  }
  if (L->in_features % 128)
    return fail(PARO_ERR_UNSUPPORTED, "in_features=%lld: the GPU path rotates 128-channel blocks",
                (long long)L->in_features);
  if (L->krot > kMaxKrot) return fail(PARO_ERR_UNSUPPORTED, "krot=%d exceeds %d", L->krot, kMaxKrot);
  if (L->in_features > kMaxDim || L->out_features > kMaxOut)
    return fail(PARO_ERR_UNSUPPORTED, "in_features > %lld or out_features > %lld", (long long)kMaxDim,
                (long long)kMaxOut);
  return PARO_OK;
}

int check_rotation_tensors(const paro_w4_layer *L) {
  if (!L->pairs || !L->theta || !L->channel_scales)
    return fail(PARO_ERR_NULL, "pairs, theta and channel_scales are required");
  if (!aligned(L->pairs, 4) || !aligned(L->theta, 4) || !aligned(L->channel_scales, 4))
    return fail(PARO_ERR_ALIGN, "pairs, theta, channel_scales must be 4-byte aligned");
  return PARO_OK;
}

int check_weight_tensors(const paro_w4_layer *L) {
  if (!L->qweight || !L->qzeros || !L->scales) return fail(PARO_ERR_NULL, "qweight, qzeros, scales are required");
  if (!aligned(L->qweight, 16) || !aligned(L->scales, 16) || !aligned(L->qzeros, 4) ||
      (L->bias && !aligned(L->bias, 8)))
    return fail(PARO_ERR_ALIGN, "qweight/scales must be 16-byte aligned, qzeros 4, bias 8");
  return PARO_OK;
}

int check_tokens(int64_t tokens) {
  if (tokens < 0) return fail(PARO_ERR_SHAPE, "tokens=%lld is negative", (long long)tokens);
  if (tokens > kMaxTokens) return fail(PARO_ERR_UNSUPPORTED, "tokens=%lld exceeds %lld", (long long)tokens,
                                       (long long)kMaxTokens);
  return PARO_OK;
}

bool act_dtype(int dt) { return dt == PARO_F16 || dt == PARO_BF16; }

int hip_fail(hipError_t e, const char *what) {
  return fail(PARO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool overlap(const void *a, size_t an, const void *b, size_t bn) {
  const char *pa = (const char *)a, *pb = (const char *)b;
  return an && bn && pa < pb + bn && pb < pa + an;
}

paro::LinearArgs linear_args(const paro_w4_layer *L, int64_t tokens, const void *x, paro_dtype x_dt, void *y,
                             paro_dtype y_dt) {
  paro::LinearArgs a;
  a.I = L->in_features;
  a.O = L->out_features;
  a.tokens = tokens;
  a.krot = L->krot;
  a.group = (int)group_of(L);
  a.pairs = L->pairs;
  a.theta = L->theta;
  a.cs = L->channel_scales;
  a.qweight = L->qweight;
  a.qzeros = L->qzeros;
  a.scales = L->scales;
  a.bias = L->bias;
  a.x = x;
  a.x_dt = (int)x_dt;
  a.y = y;
  a.y_dt = (int)y_dt;
  a.experts = 0;
  a.expert_offsets = nullptr;
  return a;
}

// rows: one group over the whole row, whose rotation the fused decode
// prologue (one 128-channel block per wave) cannot do
paro_path auto_path(int64_t tokens, bool rows = false) {
  if (tokens <= 4 && !rows) return PARO_PATH_DECODE_FUSED;
  if (tokens <= 16) return PARO_PATH_DECODE_SPLIT;
  return PARO_PATH_PREFILL;
}

// Workspace layout: [counters kCounterBytes][x_r (split / prefill)][partials (decode) | H, L (prefill)]
// X_r in the workspace: row-major for the split decode path, the GEMM's
// 16-row tiled layout (rows padded to a multiple of 16) for prefill.
size_t xr_region(const paro_w4_layer *L, int64_t tokens, paro_path path) {
  if (path == PARO_PATH_DECODE_FUSED) return 0;
  const int64_t rows = path == PARO_PATH_PREFILL ? paro::tiled_rows(tokens) : tokens;
  return align_up((size_t)rows * (size_t)L->in_features * 2, 256);
}

size_t workspace_for(const paro_w4_layer *L, int64_t tokens, paro_path path) {
  const int64_t I = L->in_features, O = L->out_features;
  size_t bytes = kCounterBytes + xr_region(L, tokens, path);
  if (path != PARO_PATH_PREFILL)
    bytes += paro::decode_partial_bytes(paro::plan_decode(I, O, tokens, path == PARO_PATH_DECODE_FUSED, (int)group_of(L)), tokens, O);
  else if (!full_row(L))
    bytes += paro::rot_mat_bytes(I);  // the dense rotation (one group over the row is rotated stage by stage)
  return bytes;
}

}  // namespace

extern "C" {

int paro_abi_version(void) { return PARO_ABI_VERSION; }

const char *paro_last_error(void) { return g_last_error.c_str(); }

int paro_validate_layer(const paro_w4_layer *L) {
  int rc = check_method_shape(L);
  if (rc) return rc;
  if (!L->pairs) return fail(PARO_ERR_NULL, "pairs is NULL");
  const int64_t I = L->in_features, G = group_of(L);
  if (G > 32768) return fail(PARO_ERR_SHAPE, "group_size=%lld exceeds int16 pair indices", (long long)G);
  std::vector<unsigned char> seen((size_t)G);
  for (int t = 0; t < L->krot; ++t) {
    for (int64_t g = 0; g < I / G; ++g) {
      std::fill(seen.begin(), seen.end(), 0);
      for (int64_t e = 0; e < G; ++e) {
        const int v = L->pairs[(int64_t)t * I + g * G + e];
        if (v < 0 || v >= G || seen[(size_t)v])
          return fail(PARO_ERR_PAIRS, "pairs[%d][%lld] = %d: stage %d group %lld is not a permutation of 0..%lld",
                      t, (long long)(g * G + e), v, t, (long long)g, (long long)(G - 1));
        seen[(size_t)v] = 1;
      }
    }
  }
  return ok();
}

int paro_scale_rotate(const paro_w4_layer *L, const void *x, paro_dtype x_dt, int64_t tokens, void *x_r,
                      paro_dtype xr_dt, void *stream) {
  int rc = check_gpu_shape(L, true);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (!act_dtype(xr_dt) && xr_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "x_r dtype %d invalid", (int)xr_dt);
  if (tokens == 0) return ok();
  if (!x || !x_r) return fail(PARO_ERR_NULL, "x and x_r are required");
  rc = check_rotation_tensors(L);
  if (rc) return rc;
  if (!aligned(x, 16) || !aligned(x_r, 16)) return fail(PARO_ERR_ALIGN, "x and x_r must be 16-byte aligned");
  const int64_t I = L->in_features;
  const size_t xb = (size_t)tokens * I * 2, ob = (size_t)tokens * I * (xr_dt == PARO_F32 ? 4 : 2);
  const char *xs = (const char *)x, *os = (const char *)x_r;
  const bool overlap = xs < os + ob && os < xs + xb;
  if (overlap && !(x == x_r && x_dt == xr_dt))
    return fail(PARO_ERR_SHAPE, "x_r overlaps x (only exact in-place with equal dtypes is allowed)");
  hipError_t e = full_row(L) ? paro::launch_scale_rotate_full((const uint16_t *)x, (int)x_dt, x_r, (int)xr_dt, false,
                                                               tokens, I, L->pairs, L->theta, L->channel_scales,
                                                               L->krot, (hipStream_t)stream)
                             : paro::launch_scale_rotate((const uint16_t *)x, (int)x_dt, x_r, (int)xr_dt, tokens, I,
                                                         L->pairs, L->theta, L->channel_scales, L->krot,
                                                         (int)group_of(L), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "scale_rotate launch");
  return ok();
}

size_t paro_tiled_bytes(const paro_w4_layer *L, int64_t tokens) {
  if (!L || tokens <= 0 || L->in_features <= 0) return 0;
  return (size_t)paro::tiled_rows(tokens) * (size_t)L->in_features * 2;
}

size_t paro_rotation_matrix_bytes(const paro_w4_layer *L) {
  if (!L || L->in_features <= 0) return 0;
  return paro::rot_mat_bytes(L->in_features);
}

int paro_rotation_matrix(const paro_w4_layer *L, paro_dtype x_dt, void *hl, void *stream) {
  int rc = check_gpu_shape(L);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (!hl) return fail(PARO_ERR_NULL, "hl is required");
  rc = check_rotation_tensors(L);
  if (rc) return rc;
  if (!aligned(hl, 16)) return fail(PARO_ERR_ALIGN, "hl must be 16-byte aligned");
  hipError_t e = paro::launch_rot_build((int)x_dt, L->in_features, L->pairs, L->theta, L->channel_scales, L->krot,
                                        (int)group_of(L), (uint16_t *)hl, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rotation matrix launch");
  return ok();
}

int paro_scale_rotate_tiled(const paro_w4_layer *L, const void *hl, const void *x, paro_dtype x_dt, int64_t tokens,
                            void *x_t, void *stream) {
  int rc = check_gpu_shape(L);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (tokens == 0) return ok();
  if (!hl || !x || !x_t) return fail(PARO_ERR_NULL, "hl, x and x_t are required");
  if (!aligned(hl, 16) || !aligned(x, 16) || !aligned(x_t, 16))
    return fail(PARO_ERR_ALIGN, "hl, x and x_t must be 16-byte aligned");
  const int64_t I = L->in_features;
  const size_t xb = (size_t)tokens * I * 2, tb = paro_tiled_bytes(L, tokens), hb = paro::rot_mat_bytes(I);
  const char *xs = (const char *)x, *ts = (const char *)x_t, *hs = (const char *)hl;
  if (xs < ts + tb && ts < xs + xb) return fail(PARO_ERR_SHAPE, "x_t overlaps x");
  if (hs < ts + tb && ts < hs + hb) return fail(PARO_ERR_SHAPE, "x_t overlaps hl");
  hipError_t e = paro::launch_rot_apply((const uint16_t *)x, (int)x_dt, (uint16_t *)x_t, tokens, I,
                                        (const uint16_t *)hl, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "scale_rotate_tiled launch");
  return ok();
}

int paro_w4a16_linear_tiled(const paro_w4_layer *L, const void *x_t, paro_dtype x_dt, int64_t tokens, void *y,
                            paro_dtype y_dt, void *stream) {
  int rc = check_gpu_shape(L, true);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (y_dt != x_dt && y_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "y dtype %d must equal x dtype or F32", (int)y_dt);
  if (tokens == 0) return ok();
  if (!x_t || !y) return fail(PARO_ERR_NULL, "x_t and y are required");
  rc = check_weight_tensors(L);
  if (rc) return rc;
  if (!aligned(x_t, 16) || !aligned(y, 16)) return fail(PARO_ERR_ALIGN, "x_t and y must be 16-byte aligned");
  const int64_t O = L->out_features;
  const size_t tb = paro_tiled_bytes(L, tokens), yb = (size_t)tokens * O * (y_dt == PARO_F32 ? 4 : 2);
  const char *ts = (const char *)x_t, *ys = (const char *)y;
  if (ts < ys + yb && ys < ts + tb) return fail(PARO_ERR_SHAPE, "y overlaps x_t");
  paro::LinearArgs a = linear_args(L, tokens, x_t, x_dt, y, y_dt);
  hipError_t e = paro::launch_prefill_gemm(a, (const uint16_t *)x_t, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill GEMM launch");
  return ok();
}

int paro_w4a16_linear_tiled_multi(const paro_w4_layer *layers, int n_layers, const void *const *x_t,
                                  paro_dtype x_dt, int64_t tokens, void *const *y, paro_dtype y_dt, void *stream) {
  if (!layers || !x_t || !y) return fail(PARO_ERR_NULL, "layers, x_t and y are required");
  if (n_layers < 1 || n_layers > paro::kMaxMultiLayers)
    return fail(PARO_ERR_SHAPE, "n_layers=%d must be in 1..%d", n_layers, paro::kMaxMultiLayers);
  const paro_w4_layer *L0 = &layers[0];
  int rc = PARO_OK;
  for (int i = 0; i < n_layers; ++i) {
    const paro_w4_layer *L = &layers[i];
    if ((rc = check_gpu_shape(L, true))) return rc;
    if (L->in_features != L0->in_features || group_of(L) != group_of(L0))
      return fail(PARO_ERR_SHAPE, "layer %d: in_features and group size must equal layer 0's", i);
  }
  if ((rc = check_tokens(tokens))) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (y_dt != x_dt && y_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "y dtype %d must equal x dtype or F32", (int)y_dt);
  if (tokens == 0) return ok();
  const size_t tb = paro_tiled_bytes(L0, tokens);
  auto yb = [&](int i) { return (size_t)tokens * layers[i].out_features * (y_dt == PARO_F32 ? 4 : 2); };
  for (int i = 0; i < n_layers; ++i) {
    if (!x_t[i] || !y[i]) return fail(PARO_ERR_NULL, "layer %d: x_t and y are required", i);
    if ((rc = check_weight_tensors(&layers[i]))) return rc;
    if (!aligned(x_t[i], 16) || !aligned(y[i], 16))
      return fail(PARO_ERR_ALIGN, "layer %d: x_t and y must be 16-byte aligned", i);
  }
  for (int i = 0; i < n_layers; ++i)
    for (int j = 0; j < n_layers; ++j) {
      if (overlap(y[i], yb(i), x_t[j], tb)) return fail(PARO_ERR_SHAPE, "the output of layer %d overlaps x_t of %d", i, j);
      if (j < i && overlap(y[i], yb(i), y[j], yb(j)))
        return fail(PARO_ERR_SHAPE, "the outputs of layers %d and %d overlap", j, i);
    }
  paro::LinearArgs a = linear_args(L0, tokens, x_t[0], x_dt, y[0], y_dt);
  paro::LayerTable lt{};
  lt.n = n_layers;
  for (int i = 0; i < n_layers; ++i) {
    lt.qweight[i] = layers[i].qweight;
    lt.qzeros[i] = layers[i].qzeros;
    lt.scales[i] = layers[i].scales;
    lt.bias[i] = layers[i].bias;
    lt.xt[i] = (const uint16_t *)x_t[i];
    lt.y[i] = y[i];
    lt.o[i] = layers[i].out_features;
  }
  const hipError_t e = paro::launch_prefill_gemm_multi(a, lt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill GEMM launch");
  return ok();
}

int paro_w4_unpack_dequant(const paro_w4_layer *L, uint8_t *q_out, uint8_t *z_out, void *w_out, paro_dtype w_dt,
                           void *stream) {
  int rc = check_gpu_shape(L, true);
  if (rc) return rc;
  if (w_out && !act_dtype(w_dt) && w_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "w dtype %d invalid", (int)w_dt);
  if (!q_out && !z_out && !w_out) return ok();
  rc = check_weight_tensors(L);
  if (rc) return rc;
  if ((q_out && !aligned(q_out, 8)) || (z_out && !aligned(z_out, 8)) || (w_out && !aligned(w_out, 16)))
    return fail(PARO_ERR_ALIGN, "q_out/z_out must be 8-byte and w_out 16-byte aligned");
  hipError_t e = paro::launch_unpack_dequant(L->qweight, L->qzeros, L->scales, L->in_features, L->out_features,
                                             group_of(L), q_out, z_out, w_out, (int)w_dt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "unpack_dequant launch");
  return ok();
}

int paro_w4_quantize_pack(const paro_w4_layer *L, const void *w, paro_dtype w_dt, int symmetric, int32_t *qweight,
                          int32_t *qzeros, uint16_t *scales, void *stream) {
  int rc = check_gpu_shape(L);
  if (rc) return rc;
  if (!act_dtype(w_dt) && w_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "w dtype %d invalid", (int)w_dt);
  if (!w || !qweight || !qzeros || !scales) return fail(PARO_ERR_NULL, "w, qweight, qzeros and scales are required");
  rc = check_rotation_tensors(L);
  if (rc) return rc;
  if (!aligned(w, w_dt == PARO_F32 ? 8 : 4) || !aligned(qweight, 4) || !aligned(qzeros, 4) || !aligned(scales, 2))
    return fail(PARO_ERR_ALIGN, "w must be 4-byte (8 for F32) and qweight/qzeros/scales 4/4/2-byte aligned");
  const int64_t I = L->in_features, O = L->out_features, G = group_of(L);
  const size_t wb = (size_t)I * O * (w_dt == PARO_F32 ? 4 : 2);
  const char *ws = (const char *)w;
  const char *outs[3] = {(const char *)qweight, (const char *)qzeros, (const char *)scales};
  // the kernel writes qzeros [I/G][O/8] int32 and scales [I/G][O] fp16
  const size_t outb[3] = {(size_t)I * O / 2, (size_t)(I / G) * O / 2, (size_t)(I / G) * O * 2};
  for (int i = 0; i < 3; ++i) {
    if (ws < outs[i] + outb[i] && outs[i] < ws + wb) return fail(PARO_ERR_SHAPE, "an output overlaps w");
    for (int j = 0; j < i; ++j)
      if (outs[j] < outs[i] + outb[i] && outs[i] < outs[j] + outb[j])
        return fail(PARO_ERR_SHAPE, "qweight, qzeros and scales must not overlap");
  }
  hipError_t e = paro::launch_quantize_pack(w, (int)w_dt, symmetric != 0, O, I, L->pairs, L->theta,
                                            L->channel_scales, L->krot, (int)group_of(L), qweight, qzeros, scales,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_pack launch");
  return ok();
}

int paro_scale_rotate_backward(const paro_w4_layer *L, const void *x, paro_dtype x_dt, const void *g,
                               paro_dtype g_dt, int64_t tokens, void *gx, paro_dtype gx_dt, float *gtheta,
                               float *gcs, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_gpu_shape(L);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (g_dt != PARO_F32 && g_dt != x_dt) return fail(PARO_ERR_DTYPE, "g dtype %d must be F32 or x's", (int)g_dt);
  if (gx_dt != PARO_F32 && gx_dt != x_dt) return fail(PARO_ERR_DTYPE, "gx dtype %d must be F32 or x's", (int)gx_dt);
  if (!gtheta || !gcs) return fail(PARO_ERR_NULL, "gtheta and gcs are required");
  if (tokens > 0 && (!x || !g || !gx)) return fail(PARO_ERR_NULL, "x, g and gx are required");
  rc = check_rotation_tensors(L);
  if (rc) return rc;
  const int64_t I = L->in_features;
  const size_t need = paro::rot_backward_partial_bytes(tokens, I, L->krot);
  if (!workspace || workspace_bytes < need)
    return fail(PARO_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                need);
  if (!aligned(workspace, 16) || !aligned(gtheta, 4) || !aligned(gcs, 4) ||
      (tokens > 0 && (!aligned(x, 16) || !aligned(g, 16) || !aligned(gx, 16))))
    return fail(PARO_ERR_ALIGN, "x, g, gx and the workspace must be 16-byte and gtheta/gcs 4-byte aligned");
  const size_t n = (size_t)tokens * I;
  struct Region {
    const void *p;
    size_t bytes;
  };
  const Region in[2] = {{x, n * 2}, {g, n * (g_dt == PARO_F32 ? 4 : 2)}};
  const Region out[4] = {{gx, n * (gx_dt == PARO_F32 ? 4 : 2)},
                         {gtheta, (size_t)L->krot * (I / 2) * 4},
                         {gcs, (size_t)I * 4},
                         {workspace, need}};
  auto overlap = [](const Region &a, const Region &b) {
    const char *pa = (const char *)a.p, *pb = (const char *)b.p;
    return a.bytes && b.bytes && pa < pb + b.bytes && pb < pa + a.bytes;
  };
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlap(out[i], in[j])) return fail(PARO_ERR_SHAPE, "an output or the workspace overlaps x or g");
    for (int j = 0; j < i; ++j)
      if (overlap(out[i], out[j])) return fail(PARO_ERR_SHAPE, "gx, gtheta, gcs and the workspace must not overlap");
  }
  hipError_t e = paro::launch_rot_backward(x, (int)x_dt, g, (int)g_dt, tokens, I, L->pairs, L->theta,
                                           L->channel_scales, L->krot, (int)group_of(L), gx, (int)gx_dt, gtheta, gcs,
                                           (float *)workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "scale_rotate_backward launch");
  return ok();
}

size_t paro_scale_rotate_backward_workspace_bytes(const paro_w4_layer *L, int64_t tokens) {
  if (!L || tokens < 0 || tokens > kMaxTokens || check_gpu_shape(L)) return 0;
  return paro::rot_backward_partial_bytes(tokens, L->in_features, L->krot);  // > 0 even for 0 tokens
}

}  // extern "C"

namespace {

constexpr int64_t kMxMaxBytes = (int64_t(1) << 31) - 1;  // 32-bit buffer offsets in the FP4 GEMM

int check_mx_rows(int64_t rows, int64_t I) {
  if (rows < 0) return fail(PARO_ERR_SHAPE, "rows=%lld is negative", (long long)rows);
  if (rows * (I / 2) > kMxMaxBytes)
    return fail(PARO_ERR_UNSUPPORTED, "rows * in_features / 2 = %lld exceeds %lld", (long long)(rows * (I / 2)),
                (long long)kMxMaxBytes);
  return PARO_OK;
}

int mx_quantize_weight_impl(const paro_w4_layer *L, const void *w, paro_dtype w_dt, uint8_t *codes,
                            uint8_t *scales, void *stream) {
  int rc = check_gpu_shape(L);
  if (rc) return rc;
  const int64_t I = L->in_features, rows = L->out_features;
  rc = check_mx_rows(rows, I);
  if (rc) return rc;
  if (!act_dtype(w_dt) && w_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "w dtype %d invalid", (int)w_dt);
  if (!w || !codes || !scales) return fail(PARO_ERR_NULL, "w, codes and scales are required");
  rc = check_rotation_tensors(L);
  if (rc) return rc;
  if (!aligned(w, w_dt == PARO_F32 ? 8 : 4) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(PARO_ERR_ALIGN, "w 4-byte (8 for F32), codes 16-byte and scales 4-byte aligned");
  const size_t wb = (size_t)rows * I * (w_dt == PARO_F32 ? 4 : 2), cb = (size_t)rows * I / 2,
               scb = (size_t)rows * I / 32;
  if (overlap(codes, cb, w, wb) || overlap(scales, scb, w, wb) || overlap(codes, cb, scales, scb))
    return fail(PARO_ERR_SHAPE, "codes, scales and w must not overlap");
  hipError_t e = paro::launch_mx_quantize_weight(w, (int)w_dt, rows, I, L->pairs, L->theta, L->channel_scales,
                                                 L->krot, (int)group_of(L), codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mxfp4 weight quantize launch");
  return ok();
}

int mx_gemm_checks(const uint8_t *ac, const uint8_t *as, int64_t tokens, const uint8_t *wc, const uint8_t *ws,
                   int64_t O, int64_t I, const uint16_t *bias, void *y, paro_dtype y_dt) {
  if (I <= 0 || I % 128 || O <= 0 || O % 8)
    return fail(PARO_ERR_SHAPE, "in_features %% 128 == 0 and out_features %% 8 == 0 required");
  int rc = check_mx_rows(tokens, I);
  if (!rc) rc = check_mx_rows(O, I);
  if (rc) return rc;
  if (y_dt != PARO_F16 && y_dt != PARO_BF16 && y_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "y dtype %d invalid", (int)y_dt);
  if (tokens == 0) return PARO_OK;
  if (!ac || !as || !wc || !ws || !y) return fail(PARO_ERR_NULL, "codes, scales and y are required");
  if (!aligned(ac, 16) || !aligned(wc, 16) || !aligned(as, 4) || !aligned(ws, 4) || !aligned(y, 4) ||
      (bias && !aligned(bias, 2)))
    return fail(PARO_ERR_ALIGN, "codes 16-byte, scales and y 4-byte aligned");
  const size_t yb = (size_t)tokens * O * (y_dt == PARO_F32 ? 4 : 2);
  const void *ins[5] = {ac, as, wc, ws, bias};
  const size_t inb[5] = {(size_t)tokens * I / 2, (size_t)tokens * I / 32, (size_t)O * I / 2, (size_t)O * I / 32,
                         bias ? (size_t)O * 2 : 0};
  for (int i = 0; i < 5; ++i)
    if (overlap(y, yb, ins[i], inb[i])) return fail(PARO_ERR_SHAPE, "y overlaps an input");
  return PARO_OK;
}

size_t mx_codes_region(int64_t tokens, int64_t I) { return align_up((size_t)tokens * I / 2, 256); }

}  // namespace

extern "C" {

int paro_mxfp4_quantize_weight(const paro_w4_layer *L, const void *w, paro_dtype w_dt, uint8_t *codes,
                               uint8_t *scales, void *stream) {
  return mx_quantize_weight_impl(L, w, w_dt, codes, scales, stream);
}

size_t paro_mxfp4_activation_workspace_bytes(const paro_w4_layer *L) {
  if (!L || check_gpu_shape(L)) return 0;
  return align_up(paro::rot_mat_bytes(L->in_features), 256);
}

}  // extern "C"

namespace {

// hl_pre: a caller-built rotation matrix (paro_rotation_matrix), or NULL to
// build it into the workspace.
int mx_quantize_activations_impl(const paro_w4_layer *L, const void *hl_pre, const void *x, paro_dtype x_dt,
                                 int64_t tokens, uint8_t *codes, uint8_t *scales, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  int rc = check_gpu_shape(L);
  if (rc) return rc;
  const int64_t I = L->in_features;
  rc = check_mx_rows(tokens, I);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (tokens == 0) return ok();
  if (!x || !codes || !scales) return fail(PARO_ERR_NULL, "x, codes and scales are required");
  size_t need = 0;
  if (!hl_pre) {
    rc = check_rotation_tensors(L);
    if (rc) return rc;
    need = paro_mxfp4_activation_workspace_bytes(L);
    if (!workspace || workspace_bytes < need)
      return fail(PARO_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                  need);
  }
  const void *mat = hl_pre ? hl_pre : workspace;  // where the rotation matrix is read
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(mat, 16))
    return fail(PARO_ERR_ALIGN, "x, codes and workspace (or hl) 16-byte, scales 4-byte aligned");
  const size_t xb = (size_t)tokens * I * 2, cb = (size_t)tokens * I / 2, sb = (size_t)tokens * I / 32;
  const size_t mb = hl_pre ? paro::rot_mat_bytes(I) : need;
  if (overlap(codes, cb, x, xb) || overlap(scales, sb, x, xb) || overlap(codes, cb, scales, sb) ||
      overlap(mat, mb, codes, cb) || overlap(mat, mb, scales, sb) || (!hl_pre && overlap(mat, mb, x, xb)))
    return fail(PARO_ERR_SHAPE, "x, codes, scales and the workspace (or hl) must not overlap");
  hipStream_t st = (hipStream_t)stream;
  if (!hl_pre) {
    hipError_t e = paro::launch_rot_build((int)x_dt, I, L->pairs, L->theta, L->channel_scales, L->krot,
                                          (int)group_of(L), (uint16_t *)workspace, st);
    if (e != hipSuccess) return hip_fail(e, "rotation matrix launch");
  }
  hipError_t e = paro::launch_rot_apply_mx((const uint16_t *)x, (int)x_dt, tokens, I, (const uint16_t *)mat, codes,
                                           scales, st);
  if (e != hipSuccess) return hip_fail(e, "mxfp4 activation launch");
  return ok();
}

size_t mx_linear_workspace(const paro_w4_layer *L, int64_t tokens, bool prepared) {
  if (!L || tokens <= 0 || check_gpu_shape(L)) return 0;
  return mx_codes_region(tokens, L->in_features) + align_up((size_t)tokens * L->in_features / 32, 256) +
         (prepared ? 0 : paro_mxfp4_activation_workspace_bytes(L));
}

int mx_linear_impl(const paro_w4_layer *L, const void *hl_pre, const uint8_t *w_codes, const uint8_t *w_scales,
                   const void *x, paro_dtype x_dt, int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                   size_t workspace_bytes, void *stream) {
  int rc = check_gpu_shape(L);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  const int64_t I = L->in_features, O = L->out_features;
  if (tokens == 0) return ok();
  const size_t need = mx_linear_workspace(L, tokens, hl_pre != nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(PARO_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                need);
  if (!aligned(workspace, 16)) return fail(PARO_ERR_ALIGN, "workspace must be 16-byte aligned");
  uint8_t *ac = (uint8_t *)workspace, *as = ac + mx_codes_region(tokens, I);
  uint8_t *hl = as + align_up((size_t)tokens * I / 32, 256);
  rc = mx_gemm_checks(ac, as, tokens, w_codes, w_scales, O, I, L->bias, y, y_dt);
  if (rc) return rc;
  const size_t yb = (size_t)tokens * O * (y_dt == PARO_F32 ? 4 : 2), xb = (size_t)tokens * I * 2;
  if (overlap(y, yb, x, xb) || overlap(workspace, need, x, xb) || overlap(workspace, need, y, yb))
    return fail(PARO_ERR_SHAPE, "x, y and the workspace must not overlap");
  if (hl_pre && (overlap(hl_pre, paro::rot_mat_bytes(I), workspace, need) ||
                 overlap(hl_pre, paro::rot_mat_bytes(I), y, yb)))
    return fail(PARO_ERR_SHAPE, "hl must not overlap y or the workspace");
  rc = mx_quantize_activations_impl(L, hl_pre, x, x_dt, tokens, ac, as, hl_pre ? nullptr : hl,
                                    hl_pre ? 0 : paro_mxfp4_activation_workspace_bytes(L), stream);
  if (rc) return rc;
  hipError_t e = paro::launch_mx_gemm(ac, as, tokens, w_codes, w_scales, O, I, L->bias, y, (int)y_dt,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mxfp4 GEMM launch");
  return ok();
}

}  // namespace

extern "C" {

int paro_mxfp4_quantize_activations(const paro_w4_layer *L, const void *x, paro_dtype x_dt, int64_t tokens,
                                    uint8_t *codes, uint8_t *scales, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  return mx_quantize_activations_impl(L, nullptr, x, x_dt, tokens, codes, scales, workspace, workspace_bytes,
                                      stream);
}

int paro_mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, int64_t tokens, const uint8_t *w_codes,
                    const uint8_t *w_scales, int64_t out_features, int64_t in_features, const uint16_t *bias,
                    void *y, paro_dtype y_dt, void *stream) {
  int rc = mx_gemm_checks(a_codes, a_scales, tokens, w_codes, w_scales, out_features, in_features, bias, y, y_dt);
  if (rc) return rc;
  if (tokens == 0) return ok();
  hipError_t e = paro::launch_mx_gemm(a_codes, a_scales, tokens, w_codes, w_scales, out_features, in_features, bias,
                                      y, (int)y_dt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mxfp4 GEMM launch");
  return ok();
}

size_t paro_mxfp4_linear_workspace_bytes(const paro_w4_layer *L, int64_t tokens) {
  return mx_linear_workspace(L, tokens, false);
}

int paro_mxfp4_linear(const paro_w4_layer *L, const uint8_t *w_codes, const uint8_t *w_scales, const void *x,
                      paro_dtype x_dt, int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return mx_linear_impl(L, nullptr, w_codes, w_scales, x, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream);
}

size_t paro_mxfp4_linear_prepared_workspace_bytes(const paro_w4_layer *L, int64_t tokens) {
  return mx_linear_workspace(L, tokens, true);
}

int paro_mxfp4_linear_prepared(const paro_w4_layer *L, const void *hl, const uint8_t *w_codes,
                               const uint8_t *w_scales, const void *x, paro_dtype x_dt, int64_t tokens, void *y,
                               paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream) {
  if (!hl) return fail(PARO_ERR_NULL, "hl is required");
  return mx_linear_impl(L, hl, w_codes, w_scales, x, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream);
}

paro_path paro_w4a16_linear_choose_path(const paro_w4_layer *L, int64_t tokens) {
  return auto_path(tokens, L && full_row(L));
}

size_t paro_w4a16_linear_workspace_bytes(const paro_w4_layer *L, int64_t tokens, paro_dtype x_dt,
                                         paro_path path) {
  (void)x_dt;
  if (!L || tokens <= 0 || check_gpu_shape(L, true)) return 0;
  if (path == PARO_PATH_AUTO) path = auto_path(tokens, full_row(L));
  return workspace_for(L, tokens, path);
}

}  // extern "C"

namespace {

// Shared body of the linear entry points.  prerotated: x already holds X_r.
constexpr int kMaxExperts = 1024;  // each workgroup scans the expert offsets once

// hl_pre: the layer's dense rotation prebuilt by paro_rotation_matrix (for
// x_dt), used by the prefill path instead of building it in the workspace.
int linear_impl(const paro_w4_layer *L, const void *x, paro_dtype x_dt, int64_t tokens, void *y,
                paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream, paro_path path,
                bool prerotated, int experts = 0, const int64_t *expert_offsets = nullptr,
                const void *hl_pre = nullptr) {
  const bool rows = full_row(L);
  int rc = check_gpu_shape(L, !hl_pre && experts == 0);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (y_dt != x_dt && y_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "y dtype %d must equal x dtype or F32", (int)y_dt);
  if (path < PARO_PATH_AUTO || path > PARO_PATH_PREFILL) return fail(PARO_ERR_SHAPE, "unknown path %d", (int)path);
  if (prerotated && path == PARO_PATH_DECODE_FUSED)
    return fail(PARO_ERR_SHAPE, "the fused decode path rotates itself; use AUTO, DECODE_SPLIT or PREFILL");
  if (experts != 0) {
    if (experts < 0 || experts > kMaxExperts)
      return fail(PARO_ERR_SHAPE, "num_experts=%d must be in 1..%d", experts, kMaxExperts);
    if (!expert_offsets) return fail(PARO_ERR_NULL, "expert_offsets is required");
    if (!aligned(expert_offsets, 8)) return fail(PARO_ERR_ALIGN, "expert_offsets must be 8-byte aligned");
    path = PARO_PATH_PREFILL;  // the grouped GEMM runs on the prefill kernel
  }
  if (rows && path == PARO_PATH_DECODE_FUSED)
    return fail(PARO_ERR_UNSUPPORTED, "one group over the whole row: the fused decode path rotates 128-channel "
                                      "blocks; use AUTO, DECODE_SPLIT or PREFILL");
  if (tokens == 0) return ok();
  if (path == PARO_PATH_AUTO) {
    path = auto_path(tokens, rows);
    if (prerotated && path == PARO_PATH_DECODE_FUSED) path = PARO_PATH_DECODE_SPLIT;
  }
  if ((path == PARO_PATH_DECODE_FUSED || path == PARO_PATH_DECODE_SPLIT) && tokens > 16)
    return fail(PARO_ERR_UNSUPPORTED, "decode paths take at most 16 tokens (got %lld)", (long long)tokens);
  if (!x || !y) return fail(PARO_ERR_NULL, "x and y are required");
  rc = prerotated ? PARO_OK : check_rotation_tensors(L);
  if (!rc) rc = check_weight_tensors(L);
  if (rc) return rc;
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(PARO_ERR_ALIGN, "x and y must be 16-byte aligned");
  const int64_t I = L->in_features, O = L->out_features;
  {
    const char *xs = (const char *)x, *ys = (const char *)y;
    const size_t xb = (size_t)tokens * I * 2, yb = (size_t)tokens * O * (y_dt == PARO_F32 ? 4 : 2);
    if (xs < ys + yb && ys < xs + xb) return fail(PARO_ERR_SHAPE, "y overlaps x");
  }
  const bool prebuilt = hl_pre && path == PARO_PATH_PREFILL && !prerotated;
  if (prebuilt && !aligned(hl_pre, 16)) return fail(PARO_ERR_ALIGN, "the rotation matrix must be 16-byte aligned");
  const size_t need = prebuilt ? kCounterBytes + xr_region(L, tokens, path) : workspace_for(L, tokens, path);
  if (need > 0) {
    if (!workspace) return fail(PARO_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(PARO_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(PARO_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t xb = (size_t)tokens * I * 2, yb = (size_t)tokens * O * (y_dt == PARO_F32 ? 4 : 2);
    if (overlap(workspace, need, x, xb) || overlap(workspace, need, y, yb))
      return fail(PARO_ERR_SHAPE, "the workspace overlaps x or y");
    if (prebuilt && overlap(workspace, need, hl_pre, paro::rot_mat_bytes(I)))
      return fail(PARO_ERR_SHAPE, "the workspace overlaps the rotation matrix");
  }

  paro::LinearArgs a = linear_args(L, tokens, x, x_dt, y, y_dt);
  a.experts = experts;
  a.expert_offsets = expert_offsets;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;

  uint32_t *counters = (uint32_t *)workspace;
  char *xr = (char *)workspace + kCounterBytes;
  float *partials = (float *)(xr + xr_region(L, tokens, path));
  if (path == PARO_PATH_DECODE_FUSED) {
    const paro::DecodePlan p = paro::plan_decode(I, O, tokens, true, a.group);
    e = paro::launch_decode(a, p, nullptr, counters, partials, st);
    if (e != hipSuccess) return hip_fail(e, "decode (fused) launch");
    return ok();
  }
  if (path == PARO_PATH_DECODE_SPLIT) {  // row-major X_r into the workspace, then the split-K GEMV over it
    const void *xin = x;
    if (!prerotated) {
      e = rows ? paro::launch_scale_rotate_full((const uint16_t *)x, (int)x_dt, xr, (int)x_dt, false, tokens, I,
                                                L->pairs, L->theta, L->channel_scales, L->krot, st)
               : paro::launch_scale_rotate((const uint16_t *)x, (int)x_dt, xr, (int)x_dt, tokens, I, L->pairs,
                                           L->theta, L->channel_scales, L->krot, a.group, st);
      if (e != hipSuccess) return hip_fail(e, "scale_rotate launch");
      xin = xr;
    }
    const paro::DecodePlan p = paro::plan_decode(I, O, tokens, false, a.group);
    e = paro::launch_decode(a, p, xin, counters, partials, st);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
  }
  // prefill: X_r in the tiled layout (the dense rotation built into the
  // workspace and applied on the matrix cores, or the caller's row-major X_r
  // re-tiled), then the GEMM
  uint16_t *xt = (uint16_t *)xr;
  if (prerotated) {
    e = paro::launch_retile((const uint16_t *)x, xt, tokens, I, st);
    if (e != hipSuccess) return hip_fail(e, "retile launch");
  } else if (rows) {  // one group over the row: staged rotation straight into the tiled layout
    e = paro::launch_scale_rotate_full((const uint16_t *)x, (int)x_dt, xt, (int)x_dt, true, tokens, I, L->pairs,
                                       L->theta, L->channel_scales, L->krot, st);
    if (e != hipSuccess) return hip_fail(e, "scale_rotate launch");
  } else {
    const uint16_t *hl = (const uint16_t *)hl_pre;
    if (!prebuilt) {
      uint16_t *hw = (uint16_t *)((char *)xr + xr_region(L, tokens, path));
      e = paro::launch_rot_build((int)x_dt, I, L->pairs, L->theta, L->channel_scales, L->krot, a.group, hw, st);
      if (e != hipSuccess) return hip_fail(e, "rotation matrix launch");
      hl = hw;
    }
    e = paro::launch_rot_apply((const uint16_t *)x, (int)x_dt, xt, tokens, I, hl, st);
    if (e != hipSuccess) return hip_fail(e, "scale_rotate launch");
  }
  e = paro::launch_prefill_gemm(a, xt, st);
  if (e != hipSuccess) return hip_fail(e, "prefill GEMM launch");
  return ok();
}

}  // namespace

extern "C" {

int paro_w4a16_linear_path(const paro_w4_layer *L, const void *x, paro_dtype x_dt, int64_t tokens, void *y,
                           paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream,
                           paro_path path) {
  return linear_impl(L, x, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream, path, false);
}

int paro_w4a16_linear_prerotated(const paro_w4_layer *L, const void *x_r, paro_dtype x_dt, int64_t tokens,
                                 void *y, paro_dtype y_dt, void *workspace, size_t workspace_bytes,
                                 void *stream, paro_path path) {
  return linear_impl(L, x_r, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream, path, true);
}

int paro_w4a16_linear(const paro_w4_layer *L, const void *x, paro_dtype x_dt, int64_t tokens, void *y,
                      paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream) {
  return paro_w4a16_linear_path(L, x, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream, PARO_PATH_AUTO);
}

int paro_w4a16_linear_prepared(const paro_w4_layer *L, const void *hl, const void *x, paro_dtype x_dt,
                               int64_t tokens, void *y, paro_dtype y_dt, void *workspace, size_t workspace_bytes,
                               void *stream) {
  if (!hl) return fail(PARO_ERR_NULL, "the prebuilt rotation matrix is required");
  return linear_impl(L, x, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream, PARO_PATH_AUTO, false, 0,
                     nullptr, hl);
}

int paro_w4a16_linear_noalloc(const paro_w4_layer *L, const void *x, paro_dtype x_dt, int64_t tokens, void *y,
                              paro_dtype y_dt, void *stream) {
  // the same checks as the workspace variant first, so that a bad call
  // touches no device state
  int rc = check_gpu_shape(L, true);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  if (tokens == 0) return ok();
  const size_t need = workspace_for(L, tokens, auto_path(tokens, full_row(L)));
  if (need > paro::kNoallocScratchBytes)
    return fail(PARO_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of workspace; the allocation-free linear holds %zu "
                "(use paro_w4a16_linear with a caller workspace)",
                need, paro::kNoallocScratchBytes);
  void *scratch = nullptr;
  const hipError_t e = paro::noalloc_scratch((hipStream_t)stream, kCounterBytes, &scratch);
  if (e == hipErrorStreamCaptureUnsupported)
    return fail(PARO_ERR_UNSUPPORTED, "the first allocation-free call on a device must not be graph-captured");
  if (e != hipSuccess) return hip_fail(e, "allocation-free scratch set-up");
  return linear_impl(L, x, x_dt, tokens, y, y_dt, scratch, paro::kNoallocScratchBytes, stream, PARO_PATH_AUTO,
                     false);
}

size_t paro_w4a16_linear_prepared_workspace_bytes(const paro_w4_layer *L, int64_t tokens) {
  if (!L || tokens <= 0 || check_gpu_shape(L)) return 0;
  const paro_path path = auto_path(tokens);
  return path == PARO_PATH_PREFILL ? kCounterBytes + xr_region(L, tokens, path) : workspace_for(L, tokens, path);
}

size_t paro_w4a16_linear_prepared_multi_workspace_bytes(const paro_w4_layer *layers, int n_layers,
                                                        int64_t tokens) {
  if (!layers || n_layers < 1 || n_layers > paro::kMaxMultiLayers || tokens <= 0) return 0;
  const paro_w4_layer *L = &layers[0];
  for (int i = 0; i < n_layers; ++i)
    if (check_gpu_shape(&layers[i])) return 0;
  const paro_path path = auto_path(tokens);
  // prefill: one tiled X_r per layer (the layers run in one GEMM launch; its
  // size depends on in_features alone); decode: the layers run one after
  // another on one workspace, the largest any of them needs
  if (path == PARO_PATH_PREFILL) return kCounterBytes + (size_t)n_layers * xr_region(L, tokens, path);
  size_t most = 0;
  for (int i = 0; i < n_layers; ++i) most = std::max(most, workspace_for(&layers[i], tokens, path));
  return most;
}

static_assert(PARO_MULTI_MAX_LAYERS == paro::kMaxMultiLayers, "the header and the kernels agree on the layer count");

int paro_w4a16_linear_prepared_multi(const paro_w4_layer *layers, int n_layers, const void *const *hl,
                                     const void *x, paro_dtype x_dt, int64_t tokens, void *const *y,
                                     paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream) {
  if (!layers || !hl || !y) return fail(PARO_ERR_NULL, "layers, hl and y are required");
  if (n_layers < 1 || n_layers > paro::kMaxMultiLayers)
    return fail(PARO_ERR_SHAPE, "n_layers=%d must be in 1..%d", n_layers, paro::kMaxMultiLayers);
  const paro_w4_layer *L0 = &layers[0];
  int rc = check_gpu_shape(L0);
  if (!rc) rc = check_tokens(tokens);
  if (rc) return rc;
  for (int i = 0; i < n_layers; ++i) {
    const paro_w4_layer *L = &layers[i];
    if ((rc = check_gpu_shape(L))) return rc;
    if (L->in_features != L0->in_features || group_of(L) != group_of(L0) || L->krot != L0->krot)
      return fail(PARO_ERR_SHAPE, "layer %d: in_features, group size and krot must equal layer 0's", i);
    if (!hl[i] || !y[i]) return fail(PARO_ERR_NULL, "layer %d: hl and y are required", i);
  }
  if (!act_dtype(x_dt)) return fail(PARO_ERR_DTYPE, "x dtype %d must be F16 or BF16", (int)x_dt);
  if (y_dt != x_dt && y_dt != PARO_F32) return fail(PARO_ERR_DTYPE, "y dtype %d must equal x dtype or F32", (int)y_dt);
  if (tokens == 0) return ok();
  const paro_path path = auto_path(tokens);
  if (path != PARO_PATH_PREFILL || n_layers == 1) {
    // decode (or one layer): the single-layer call per layer, in order, on
    // one workspace (stream order keeps the calls apart)
    for (int i = 0; i < n_layers; ++i)
      if ((rc = paro_w4a16_linear_prepared(&layers[i], hl[i], x, x_dt, tokens, y[i], y_dt, workspace,
                                           workspace_bytes, stream)))
        return rc;
    return ok();
  }
  if (!x) return fail(PARO_ERR_NULL, "x is required");
  const int64_t I = L0->in_features;
  const size_t xb = (size_t)tokens * I * 2;
  auto yb = [&](int i) { return (size_t)tokens * layers[i].out_features * (y_dt == PARO_F32 ? 4 : 2); };
  const size_t hb = paro::rot_mat_bytes(I), xrb = xr_region(L0, tokens, path);
  const size_t need = kCounterBytes + (size_t)n_layers * xrb;
  if (!aligned(x, 16)) return fail(PARO_ERR_ALIGN, "x must be 16-byte aligned");
  if (!workspace) return fail(PARO_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  if (workspace_bytes < need) return fail(PARO_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(PARO_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (overlap(workspace, need, x, xb)) return fail(PARO_ERR_SHAPE, "the workspace overlaps x");
  for (int i = 0; i < n_layers; ++i) {
    const paro_w4_layer *L = &layers[i];
    if ((rc = check_rotation_tensors(L)) || (rc = check_weight_tensors(L))) return rc;
    if (!aligned(y[i], 16) || !aligned(hl[i], 16))
      return fail(PARO_ERR_ALIGN, "layer %d: y and hl must be 16-byte aligned", i);
    if (overlap(y[i], yb(i), x, xb)) return fail(PARO_ERR_SHAPE, "layer %d: y overlaps x", i);
    if (overlap(workspace, need, y[i], yb(i)) || overlap(workspace, need, hl[i], hb))
      return fail(PARO_ERR_SHAPE, "layer %d: the workspace overlaps y or hl", i);
    for (int j = 0; j < i; ++j)
      if (overlap(y[i], yb(i), y[j], yb(j))) return fail(PARO_ERR_SHAPE, "the outputs of layers %d and %d overlap", j, i);
  }
  hipStream_t st = (hipStream_t)stream;
  const void *xts[paro::kMaxMultiLayers];
  for (int i = 0; i < n_layers; ++i) {
    uint16_t *xt = (uint16_t *)((char *)workspace + kCounterBytes + (size_t)i * xrb);
    const hipError_t e = paro::launch_rot_apply((const uint16_t *)x, (int)x_dt, xt, tokens, I, (const uint16_t *)hl[i], st);
    if (e != hipSuccess) return hip_fail(e, "scale_rotate launch");
    xts[i] = xt;
  }
  return paro_w4a16_linear_tiled_multi(layers, n_layers, xts, x_dt, tokens, y, y_dt, stream);
}

int paro_w4a16_moe_linear(const paro_w4_layer *L, int num_experts, const int64_t *expert_offsets, const void *x,
                          paro_dtype x_dt, int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                          size_t workspace_bytes, void *stream) {
  if (num_experts == 0) return fail(PARO_ERR_SHAPE, "num_experts must be >= 1");
  return linear_impl(L, x, x_dt, tokens, y, y_dt, workspace, workspace_bytes, stream, PARO_PATH_PREFILL, false,
                     num_experts, expert_offsets);
}

size_t paro_w4a16_moe_linear_workspace_bytes(const paro_w4_layer *L, int64_t tokens, paro_dtype x_dt) {
  return paro_w4a16_linear_workspace_bytes(L, tokens, x_dt, PARO_PATH_PREFILL);
}

}  // extern "C"

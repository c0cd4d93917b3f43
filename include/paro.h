/*
 * paro.h - C-ABI of libparo: the rotated W4A16 linear on MI355X (gfx950).
 *
 *   Y = (X . D^-1 . R) . Q(W_r)^T + b
 *
 * computed by hand-written HIP kernels.  Notation and stored tensors follow
 * the "ParoQuant" page of the GPTQModel wiki (GPT-QModel 7.7.0):
 *   - Concepts / Pairwise Givens rotations: within each group of G input
 *     channels a stage splits the channels into disjoint pairs; a pair (a, b)
 *     with angle theta becomes (a cos + b sin, -a sin + b cos); the krot
 *     stages run in order; pair indices are local to their group.
 *   - Concepts / Activation and weight transforms: X_r = X D^-1 R, and the
 *     stored channel_scales are D^-1 (they multiply the activations);
 *     Y = X_r Q(W_r)^T + b.
 *   - Checkpoint and inference implementation / Stored tensors: qweight
 *     (I, O/8) and qzeros (I/G, O/8) AWQ-packed int32, scales (I/G, O),
 *     pairs int16 (krot, I), theta (krot, I/2), channel_scales (I), bias (O).
 *   - Triton plans and tuning: the GEMM unpacks the 4-bit tile, subtracts the
 *     zero points, multiplies by the group scales and accumulates in fp32.
 *   - "GPTQ, GPTAQ, and RTN" wiki, quantizer: x_hat = scale * (q - zero).
 *
 * Readings of points the pages leave open (the same readings the CPU oracle
 * takes, written independently there):
 *   - pairs[t][g*G + 2p] and pairs[t][g*G + 2p + 1] are the local indices of
 *     the first (a) and second (b) member of pair p of group g at stage t;
 *     theta[t][g*G/2 + p] is its angle, in radians, fp32.
 *   - AWQ word layout: bits 4s..4s+3 of qweight[k][w] hold column 8w + O(s)
 *     with O = (0,2,4,6,1,3,5,7); qzeros uses the same layout per group.
 *   - scales and bias are fp16 for every activation dtype; channel_scales is
 *     fp32.
 *
 * Conventions for every entry point below:
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch cuda memory)
 *     owned by the caller; the library allocates nothing, keeps no pointer
 *     after the call and performs no host synchronisation.  `layer` itself is
 *     a host struct read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream); the
 *     work is enqueued on it and outputs are valid once it completes.
 *   - Return value: PARO_OK or a paro_status code.  Arguments are checked on
 *     the host before anything is enqueued; on error nothing is launched and
 *     paro_last_error() (thread-local) describes the failure.  Launch errors
 *     map to PARO_ERR_HIP.  No C++ exception crosses the ABI.
 *   - GPU limits: G = 32, 64 or 128, 1 <= krot <= 64, I a multiple of 128 and <= 2^22,
 *     O a multiple of 8 and <= 2^21, tokens <= 2^21.  G = -1 (or G = I: one
 *     rotation and quantization group over the whole row; Concepts / Pairwise
 *     Givens rotations) is taken by paro_scale_rotate, the linear on its
 *     DECODE_SPLIT and PREFILL paths (AUTO picks them), the allocation-free
 *     linear, paro_w4a16_linear_prerotated / _tiled and
 *     paro_w4_unpack_dequant, with I <= 16384 (whole rows are staged in LDS);
 *     the other entry points return PARO_ERR_UNSUPPORTED for it.  x, y, x_r, w_out,
 *     qweight and scales 16-byte aligned, bias 8-byte aligned, qzeros,
 *     pairs, theta and channel_scales 4-byte aligned.  Other values give
 *     PARO_ERR_UNSUPPORTED / _SHAPE / _ALIGN.
 *   - Pair contents are NOT read on the host by the GPU entry points (they
 *     are device memory); kernels mask every pair index into its group, so
 *     an invalid schedule yields wrong numbers, never an out-of-bounds
 *     access.  paro_validate_layer() checks a host copy.
 */
#ifndef PARO_H
#define PARO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARO_ABI_VERSION 5

/* The _RANGE_MIN / _RANGE_MAX members of the two argument enums are not
 * values to pass: they widen the enums to every int32, so that the library
 * (C++) can receive any int a caller passes and reject it with a status code
 * instead of holding an out-of-range enum value. */
typedef enum {
  PARO_F16 = 0,  /* IEEE binary16 */
  PARO_BF16 = 1, /* bfloat16      */
  PARO_F32 = 2,  /* IEEE binary32 */
  PARO_DTYPE_RANGE_MIN = -2147483647 - 1,
  PARO_DTYPE_RANGE_MAX = 2147483647
} paro_dtype;

typedef enum {
  PARO_OK = 0,
  PARO_ERR_NULL = 1,        /* a required pointer is NULL                   */
  PARO_ERR_SHAPE = 2,       /* sizes inconsistent or out of range            */
  PARO_ERR_DTYPE = 3,       /* dtype not allowed for this argument           */
  PARO_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned              */
  PARO_ERR_UNSUPPORTED = 5, /* valid for the method, not on this GPU path    */
  PARO_ERR_PAIRS = 6,       /* host-side pair schedule check failed          */
  PARO_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required       */
  PARO_ERR_HIP = 8          /* a HIP runtime call or launch failed           */
} paro_status;

/* Which kernel sequence paro_w4a16_linear_path() runs. */
typedef enum {
  PARO_PATH_AUTO = 0,         /* choose by shape (what paro_w4a16_linear does)   */
  PARO_PATH_DECODE_FUSED = 1, /* one kernel: rotation in the activation-load
                                 prologue + split-K MFMA GEMV; tokens <= 16      */
  PARO_PATH_DECODE_SPLIT = 2, /* scale_rotate into the workspace, then the same
                                 GEMV reading X_r; tokens <= 16                  */
  PARO_PATH_PREFILL = 3,      /* scale_rotate into the workspace (in the GEMM's
                                 16-row tiled layout), then the MFMA GEMM with
                                 LDS-staged dequantized weight tiles            */
  PARO_PATH_RANGE_MIN = -2147483647 - 1,
  PARO_PATH_RANGE_MAX = 2147483647
} paro_path;

/* One rotated W4 linear layer: sizes plus device pointers to its tensors. */
typedef struct {
  int64_t in_features;         /* I                                          */
  int64_t out_features;        /* O                                          */
  int32_t group_size;          /* G (32, 64, 128 or -1 = I on the GPU)       */
  int32_t krot;                /* number of rotation stages                  */
  const int16_t *pairs;        /* [krot][I]   local pair indices             */
  const float *theta;          /* [krot][I/2] angles (radians)               */
  const float *channel_scales; /* [I]         D^-1                           */
  const int32_t *qweight;      /* [I][O/8]    AWQ-packed 4-bit codes         */
  const int32_t *qzeros;       /* [I/G][O/8]  AWQ-packed 4-bit zero points   */
  const uint16_t *scales;      /* [I/G][O]    fp16 group scales              */
  const uint16_t *bias;        /* [O] fp16 or NULL                           */
} paro_w4_layer;

/*
 * Channel scaling and pairwise rotation of activations ("ParoQuant" wiki,
 * Concepts / Pairwise Givens rotations and Activation and weight transforms):
 *   x_r[m][k] = ((x[m] . D^-1) . R)[k]      for m < tokens, k < I,
 * computed in fp32 and rounded to nearest even into xr_dt.
 *   x    : [tokens][I] x_dt in {F16, BF16}, row-major, contiguous.
 *   x_r  : [tokens][I] xr_dt in {F16, BF16, F32}; may alias x exactly when
 *          xr_dt == x_dt (in-place); any other overlap is not allowed.
 * Uses layer->pairs, theta, channel_scales only.  tokens == 0 is a no-op.
 */
int paro_scale_rotate(const paro_w4_layer *layer, const void *x, paro_dtype x_dt,
                      int64_t tokens, void *x_r, paro_dtype xr_dt, void *stream);

/*
 * AWQ unpack and affine dequantization of the stored weight ("ParoQuant"
 * wiki, Stored tensors and Triton plans; "GPTQ, GPTAQ, and RTN" wiki,
 * quantizer):
 *   q_out[k][n] = code of column n, row k          (uint8, [I][O])
 *   z_out[g][n] = zero point of column n, group g  (uint8, [I/G][O])
 *   w_out[k][n] = (q[k][n] - z[k/G][n]) * s[k/G][n], computed exactly and
 *                 rounded to nearest even into w_dt in {F16, BF16, F32}.
 * Any of q_out, z_out, w_out may be NULL (not written); all NULL is a no-op.
 * This materialises a dense weight for tests and for callers that want a
 * library GEMM; the linear below never materialises it.
 */
int paro_w4_unpack_dequant(const paro_w4_layer *layer, uint8_t *q_out, uint8_t *z_out,
                           void *w_out, paro_dtype w_dt, void *stream);

/*
 * The rotated W4A16 linear ("ParoQuant" wiki, Activation and weight
 * transforms; Backend reference: ParoLinear flattens leading dims, rotates,
 * applies the quantized projection and restores the shape):
 *   y[m][n] = sum_k x_r[m][k] * (q[k][n] - z[k/G][n]) * s[k/G][n] + bias[n]
 * with fp32 accumulation, bias added in fp32, one RNE rounding into y_dt.
 *   x : [tokens][I] x_dt in {F16, BF16} (leading dims flattened by caller).
 *   y : [tokens][O] y_dt == x_dt, or F32; must not overlap x.
 *   workspace / workspace_bytes : device scratch of at least
 *       paro_w4a16_linear_workspace_bytes(layer, tokens, x_dt, path) bytes,
 *       16-byte aligned.  It MUST be zero-filled before its first use with
 *       this library; every call that completes leaves its counter area zero
 *       again, so one zeroed workspace serves any number of sequential calls.
 *       Calls that overlap in time (other streams) need separate workspaces.
 * paro_w4a16_linear picks the path by shape; _path forces one (tests and
 * tuning).  Results of different paths agree to fp32-accumulation rounding;
 * each path is deterministic (a repeated call gives identical bits).
 */
int paro_w4a16_linear(const paro_w4_layer *layer, const void *x, paro_dtype x_dt,
                      int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                      size_t workspace_bytes, void *stream);
int paro_w4a16_linear_path(const paro_w4_layer *layer, const void *x, paro_dtype x_dt,
                           int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                           size_t workspace_bytes, void *stream, paro_path path);

/*
 * paro_w4a16_linear with the layer's dense rotation built once beforehand.
 * The rotation is a fixed linear map per 128-channel group ("ParoQuant" wiki,
 * Concepts / Pairwise Givens rotations: the stages compose to one orthogonal
 * map local to each group; Activation and weight transforms: D^-1 then R),
 * so R'_g = diag(cs_g) . R_g depends on the layer alone, like the packed
 * weight: paro_rotation_matrix(layer, x_dt, hl) builds it once, and every
 * later call passes it here instead of rebuilding it.
 *   hl : from paro_rotation_matrix for this layer and x_dt (I * 512 bytes,
 *        16-byte aligned, caller-owned, not written).
 * The path is chosen as by paro_w4a16_linear: many tokens run the PREFILL
 * kernels (hl applied on the matrix cores, then the GEMM); up to 16 tokens
 * run the decode kernels, which rotate stage by stage and do not read hl.
 * Results equal paro_w4a16_linear's bit for bit.  workspace: zero-filled
 * before first use as for paro_w4a16_linear, of
 * paro_w4a16_linear_prepared_workspace_bytes(layer, tokens) bytes (the
 * prefill path needs no room for the rotation matrix); it must not overlap
 * x, y or hl.  Errors as paro_w4a16_linear, plus PARO_ERR_NULL for hl and
 * PARO_ERR_ALIGN / _SHAPE for its alignment and overlaps.
 */
int paro_w4a16_linear_prepared(const paro_w4_layer *layer, const void *hl, const void *x, paro_dtype x_dt,
                               int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                               size_t workspace_bytes, void *stream);
size_t paro_w4a16_linear_prepared_workspace_bytes(const paro_w4_layer *layer, int64_t tokens);

/*
 * Several layers that read the same input, each with its own rotation,
 * packed weight, bias and output: the query, key and value projections of
 * an attention block, the gate and up projections of an MLP.  For
 * i < n_layers:
 *   y[i] = paro_w4a16_linear_prepared(&layers[i], hl[i], x, ...)
 * (page "ParoQuant", Concepts / Activation and weight transforms: every
 * layer is its own rotated linear; nothing is shared but the input x).
 *   layers   : n_layers (1..PARO_MULTI_MAX_LAYERS) host descriptors; their
 *              in_features, group_size (32, 64 or 128) and krot must be
 *              equal (PARO_ERR_SHAPE otherwise); out_features may differ.
 *   hl       : n_layers rotation matrices from paro_rotation_matrix (as
 *              for paro_w4a16_linear_prepared), caller-owned, not written.
 *   y        : n_layers outputs [tokens][their out_features] in y_dt, 16-byte
 *              aligned, not overlapping x, each other or the workspace.
 * Many tokens (the PREFILL path): each layer's input rotation runs into its
 * own tiled X_r, then ONE GEMM launch covers the output tiles of all the
 * layers, so layers too narrow to fill the chip alone (1024 outputs at 4096
 * tokens) fill it together.  Up to 16 tokens the layers run one after
 * another through the decode kernels.  Results equal those of n_layers
 * paro_w4a16_linear_prepared calls bit for bit.  workspace: zero-filled
 * before first use, of
 * paro_w4a16_linear_prepared_multi_workspace_bytes(layers, n_layers, tokens)
 * bytes (one tiled X_r per layer on the PREFILL path).  Errors as
 * paro_w4a16_linear_prepared, plus PARO_ERR_SHAPE for n_layers or
 * mismatched shapes.
 */
#define PARO_MULTI_MAX_LAYERS 4
int paro_w4a16_linear_prepared_multi(const paro_w4_layer *layers, int n_layers, const void *const *hl,
                                     const void *x, paro_dtype x_dt, int64_t tokens, void *const *y,
                                     paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream);
size_t paro_w4a16_linear_prepared_multi_workspace_bytes(const paro_w4_layer *layers, int n_layers,
                                                        int64_t tokens);

/*
 * paro_w4a16_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation with no workspace argument.  The
 * library holds the workspace itself, one device array of 64 MiB per GPU
 * (PARO_NOALLOC_SCRATCH_BYTES), kept until the process ends; the call makes
 * no allocation of any kind.  Results equal paro_w4a16_linear's bit for bit.
 *   - Shapes whose workspace (paro_w4a16_linear_workspace_bytes for the
 *     AUTO path) exceeds the scratch give PARO_ERR_UNSUPPORTED, with nothing
 *     launched: e.g. 4096 tokens of a 14336-channel input (117 MB of rotated
 *     activations).  Up to 16 tokens every supported layer fits.
 *   - The first call on a device sets its scratch up (its address, and a
 *     fill kernel on `stream` that zeroes the split-K counters); it must not
 *     be made under graph capture (PARO_ERR_UNSUPPORTED).  Later calls may
 *     be captured.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *     time on one GPU (different streams, or graphs replayed concurrently)
 *     race and give wrong results.  The scratch keeps the last call's
 *     contents; its split-K counters are left zero by every completed call.
 * Other arguments and errors as paro_w4a16_linear.
 */
#define PARO_NOALLOC_SCRATCH_BYTES (64u << 20)
int paro_w4a16_linear_noalloc(const paro_w4_layer *layer, const void *x, paro_dtype x_dt, int64_t tokens,
                              void *y, paro_dtype y_dt, void *stream);

/*
 * The quantized projection alone, over activations that are already scaled
 * and rotated (x_r, e.g. from paro_scale_rotate with xr_dt == x_dt):
 *   y[m][n] = sum_k x_r[m][k] * (q[k][n] - z[k/G][n]) * s[k/G][n] + bias[n].
 * It runs exactly the contraction kernel of the DECODE_SPLIT path (tokens <=
 * 16) or of the PREFILL path, so timing it isolates that kernel; for PREFILL
 * x_r is first copied into the GEMM's tiled layout in the workspace (a
 * separate copy kernel, one read and one write of x_r).  path must be
 * PARO_PATH_AUTO, _DECODE_SPLIT or _PREFILL; layer->pairs/theta/
 * channel_scales are not used.  Workspace as for paro_w4a16_linear (the
 * same size suffices).
 */
int paro_w4a16_linear_prerotated(const paro_w4_layer *layer, const void *x_r, paro_dtype x_dt,
                                 int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                                 size_t workspace_bytes, void *stream, paro_path path);

/*
 * Tiled X_r: the operand layout of the PREFILL contraction.  Rows are padded
 * to a multiple of 16 (pad rows are zero) and every 16-row x 32-column block
 * is 1 KB, contiguous, in the order the 64 lanes of one 16x16x32 MFMA hold
 * an A operand.  Element (m, k), m < rows, k < I, is at element index
 *     ((m/16) * (I/32) + k/32) * 512 + (((k%32)/8) * 16 + m%16) * 8 + k%8
 * (2-byte elements of the activation dtype).  paro_tiled_bytes() gives the
 * buffer size: ceil(tokens/16) * 16 * I * 2 bytes.
 */
size_t paro_tiled_bytes(const paro_w4_layer *layer, int64_t tokens);

/*
 * Dense form of the scaled rotation, per 128-channel group g ("ParoQuant"
 * wiki, Concepts / Pairwise Givens rotations: the stages compose to one
 * orthogonal map per group; Activation and weight transforms: D^-1 then R):
 *   R'_g[i][j] = ((e_i . diag(cs_g)) . R_g)[j],   i, j < 128,
 * i.e. the scaled unit rows pushed through the krot stages in fp32, stored
 * as two matrices in x_dt, H = rne(R') and L = rne(R' - H), whose sum holds
 * R' to about 2^-16 relative (BF16; 2^-22 for F16).
 *   hl : paro_rotation_matrix_bytes(layer) = I * 512 bytes, 16-byte aligned,
 *        caller-owned; layout [g][H, L][128 output channels in the order the
 *        matrix cores consume them][128 input channels].  Its contents are
 *        for paro_scale_rotate_tiled only.
 * Uses layer->pairs, theta, channel_scales; depends on the layer and x_dt,
 * not on the tokens, so one build serves every later call with that layer.
 */
size_t paro_rotation_matrix_bytes(const paro_w4_layer *layer);
int paro_rotation_matrix(const paro_w4_layer *layer, paro_dtype x_dt, void *hl, void *stream);

/*
 * paro_scale_rotate with the result written in the tiled layout above, as
 * x_t = rne(x . H + x . L) with fp32 accumulation on the matrix cores
 * (hl from paro_rotation_matrix for this layer and x_dt; x_t: x dtype,
 * 16-byte aligned, paro_tiled_bytes(layer, tokens) bytes; must not overlap
 * x or hl).  The two calls are the rotation of the PREFILL path.
 */
int paro_scale_rotate_tiled(const paro_w4_layer *layer, const void *hl, const void *x,
                            paro_dtype x_dt, int64_t tokens, void *x_t, void *stream);

/*
 * The PREFILL contraction alone over X_r in the tiled layout (for example
 * from paro_scale_rotate_tiled): y as in paro_w4a16_linear.  Needs no
 * workspace; layer->pairs/theta/channel_scales are not used.  Together the
 * two calls compute exactly what paro_w4a16_linear_path(..., PREFILL)
 * computes, and a rotated x_t can be reused by several projections that
 * share the same rotation.
 */
int paro_w4a16_linear_tiled(const paro_w4_layer *layer, const void *x_t, paro_dtype x_dt,
                            int64_t tokens, void *y, paro_dtype y_dt, void *stream);

/*
 * paro_w4a16_linear_tiled for several layers (in_features and group size
 * equal, PARO_ERR_SHAPE otherwise; out_features may differ) in ONE GEMM
 * launch over the union of their output tiles: layer i reads x_t[i] and
 * writes y[i] [tokens][its out_features] (1 <= n_layers <=
 * PARO_MULTI_MAX_LAYERS; outputs must overlap
 * no x_t and no other output).  Each y[i] equals that layer's
 * paro_w4a16_linear_tiled result bit for bit.  The GEMM of
 * paro_w4a16_linear_prepared_multi's PREFILL path.
 */
int paro_w4a16_linear_tiled_multi(const paro_w4_layer *layers, int n_layers, const void *const *x_t,
                                  paro_dtype x_dt, int64_t tokens, void *const *y, paro_dtype y_dt, void *stream);

/*
 * Mixture-of-experts projection with one rotation shared by all experts
 * ("ParoQuant" blog on the MLX port, technical notes: the experts' weights
 * are stacked into one tensor and the rotations are shared between experts).
 * The activations are scaled and rotated once for all experts, then each
 * expert's rows go through that expert's quantized projection:
 *   y[m] = x_r[m] . Q(W_e)^T + b_e   for offsets[e] <= m < offsets[e+1].
 *   layer: in_features I, out_features O, group_size (32/64/128), krot and
 *          pairs/theta/channel_scales as for paro_w4a16_linear (shared);
 *          qweight [E][I][O/8], qzeros [E][I/G][O/8], scales [E][I/G][O] and
 *          bias [E][O] (or NULL) stacked over the experts, expert-major.
 *   expert_offsets: DEVICE int64 [E+1], 8-byte aligned; rows of x are grouped
 *          by expert (the caller's routing: a token sent to k experts
 *          appears k times).  Expected nondecreasing with offsets[0] = 0 and
 *          offsets[E] = tokens; the kernels clamp them into [0, tokens] and
 *          make them nondecreasing, so malformed offsets cannot cause an
 *          out-of-bounds access, and rows outside every expert's range are
 *          not written.
 *   x [tokens][I] F16/BF16, y [tokens][O] x's dtype or F32, 16-byte aligned;
 *   workspace: paro_w4a16_moe_linear_workspace_bytes bytes, 16-byte aligned.
 * Runs on the prefill kernels (dense rotation on the matrix cores, then a
 * grouped GEMM in which each workgroup takes one 256-row tile of one
 * expert).  Errors as paro_w4a16_linear, plus PARO_ERR_SHAPE for
 * num_experts outside 1..1024 and PARO_ERR_NULL / _ALIGN for the offsets.
 */
int paro_w4a16_moe_linear(const paro_w4_layer *layer, int num_experts, const int64_t *expert_offsets,
                          const void *x, paro_dtype x_dt, int64_t tokens, void *y, paro_dtype y_dt,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes paro_w4a16_moe_linear needs (0 for 0 tokens or an invalid layer). */
size_t paro_w4a16_moe_linear_workspace_bytes(const paro_w4_layer *layer, int64_t tokens, paro_dtype x_dt);

/*
 * The offline step before the stored tensors exist: transform a dense weight
 * into the rotated domain, quantize it group-wise to four bits and pack it
 * ("ParoQuant" wiki, Concepts / Activation and weight transforms: W_r = W D R,
 * with the stored channel_scales = D^-1 dividing W's input channels;
 * Straight-through estimation: four-bit codes, symmetric codes -8..7 exported
 * with zero point 8, quantizer scales bounded to [1e-5, 1e5]; "GPTQ, GPTAQ,
 * and RTN" wiki, quantizer: q = clamp(round(x / scale) + zero, 0, 15), range
 * including zero, symmetric midpoint zero, affine zero = round(-xmin/scale),
 * finite sentinel range for all-zero groups; Stored tensors: AWQ layout).
 * Per output row n and group g of G input channels, all decisions in fp32
 * with correctly rounded division, rounding half to even.
 *   w        : [O][I] w_dt in {F16, BF16, F32}, row-major (out_features
 *              first), 4-byte aligned (8 for F32).
 *   symmetric: nonzero = symmetric (zero point 8), 0 = affine.
 *   qweight  : [I][O/8] int32 AWQ words, qzeros [I/G][O/8] int32, scales
 *              [I/G][O] fp16 bits; caller-owned device memory that must not
 *              overlap w or each other (PARO_ERR_SHAPE otherwise).
 * Uses layer->in_features, out_features, group_size, krot, pairs, theta,
 * channel_scales; layer->qweight/qzeros/scales/bias are ignored.  The outputs
 * plus the layer's rotation tensors form a layer for paro_w4a16_linear.
 */
int paro_w4_quantize_pack(const paro_w4_layer *layer, const void *w, paro_dtype w_dt, int symmetric,
                          int32_t *qweight, int32_t *qzeros, uint16_t *scales, void *stream);

/*
 * Backward of the channel scaling and the rotation, x_r = (x * cs) . R, for
 * the calibration step in which angles and channel scales are trained
 * ("ParoQuant" wiki, Straight-through estimation: optimization updates
 * angles and channel scales through the rotation; Concepts / Pairwise Givens
 * rotations for the pair formula a' = a cos + b sin, b' = -a sin + b cos).
 * With g = dL/dx_r, walking the stages back:
 *   dL/dtheta(t, p) = sum over tokens of ga' b' - gb' a'
 *   (ga, gb)        = (ga' cos - gb' sin, ga' sin + gb' cos)
 *   dL/dx           = gs * cs,  dL/dcs = sum over tokens of gs * x
 * (gs = gradient of the scaled rows x * cs).
 *   x      : [tokens][I] x_dt in {F16, BF16}, the forward's input.
 *   g      : [tokens][I] g_dt in {F32, x_dt}.
 *   gx     : [tokens][I] gx_dt in {F32, x_dt}; written.
 *   gtheta : [krot][I/2] fp32, gcs : [I] fp32; written (overwritten, not
 *            accumulated); with tokens == 0 both are zero.
 *   workspace: device memory of paro_scale_rotate_backward_workspace_bytes
 *            bytes or more (also needed for 0 tokens), 16-byte aligned: the
 *            per-group Gram matrices C = g^T x of the token splits, the dense
 *            R' = diag(cs) R and per-row partial sums of dL/dtheta.  Sums are
 *            added in a fixed order, so results are identical call to call.
 * Computed through C: dL/dtheta and dL/dcs from a walk over the 128 rows of
 * C per group, dL/dx = g . R'^T on the matrix cores.
 * x, g and gx are 16-byte aligned; no output overlaps an input, the workspace
 * or another output.  Caller-owned device memory; enqueued on `stream`.
 * Uses layer->in_features, group_size, krot, pairs, theta,
 * channel_scales.  Errors: PARO_ERR_NULL, _DTYPE, _ALIGN, _SHAPE,
 * _UNSUPPORTED, _WORKSPACE, _HIP.
 */
int paro_scale_rotate_backward(const paro_w4_layer *layer, const void *x, paro_dtype x_dt, const void *g,
                               paro_dtype g_dt, int64_t tokens, void *gx, paro_dtype gx_dt, float *gtheta,
                               float *gcs, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes paro_scale_rotate_backward needs (0 if the shape is invalid). */
size_t paro_scale_rotate_backward_workspace_bytes(const paro_w4_layer *layer, int64_t tokens);

/*
 * Four-bit activations after the rotation: the W4A4 extension in its MXFP4
 * variant ("ParoQuant" blog, Bits and formats), on the block-scaled FP4
 * matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).  Weight error
 * compensation of the GPTQ kind needs calibration data and is not done here:
 * weights are rounded to nearest.
 *
 * MXFP4 of a row of I values (OCP microscaling): blocks of 32 consecutive
 * values share an E8M0 scale byte b (2^(b - 127)), b = floor(log2 max|v|)
 * - 2 + 127 (0 for an all-zero block); each value is the E2M1 code (bit 3
 * sign; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) nearest to v / 2^(b - 127),
 * ties to the even code, clamped at 6, zero as +0.  Layout: codes [rows][I/2]
 * bytes, element 2j in the low nibble of byte j; scales [rows][I/32] bytes.
 * Decisions are taken in fp32 on the kernel's rotation of the rows (the
 * staged rotation for weights, the dense one for activations).
 *
 * Quantize the transformed weight W_r = W . D . R (w [O][I], F16/BF16/F32, 4-
 * byte aligned, 8 for F32): codes [O][I/2] (16-byte aligned), scales [O][I/32]
 * (4-byte aligned).  Uses the layer's I, O, group_size, krot, pairs, theta,
 * channel_scales.
 */
int paro_mxfp4_quantize_weight(const paro_w4_layer *layer, const void *w, paro_dtype w_dt, uint8_t *codes,
                               uint8_t *scales, void *stream);
/* Quantize the rotated activations X_r = X . D^-1 . R (x [tokens][I] F16/BF16,
 * 16-byte aligned; codes [tokens][I/2] 16-byte, scales [tokens][I/32] 4-byte
 * aligned).  The rotation runs as the dense per-group R' = diag(cs) . R on the
 * matrix cores (built into the workspace, paro_mxfp4_activation_workspace_bytes
 * bytes, 16-byte aligned) and the blocks are quantized in its epilogue. */
int paro_mxfp4_quantize_activations(const paro_w4_layer *layer, const void *x, paro_dtype x_dt, int64_t tokens,
                                    uint8_t *codes, uint8_t *scales, void *workspace, size_t workspace_bytes,
                                    void *stream);
size_t paro_mxfp4_activation_workspace_bytes(const paro_w4_layer *layer);
/* y [tokens][out_features] = A . W^T (+ bias fp16 [out_features] or NULL)
 * from MXFP4 codes and scales of A [tokens][in_features] and W
 * [out_features][in_features]; fp32 accumulation, one rounding to y_dt
 * (F16/BF16/F32).  in_features % 128 == 0, out_features % 8 == 0, and
 * rows * in_features / 2 < 2^31 for both operands. */
int paro_mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, int64_t tokens, const uint8_t *w_codes,
                    const uint8_t *w_scales, int64_t out_features, int64_t in_features, const uint16_t *bias,
                    void *y, paro_dtype y_dt, void *stream);
/* The whole W4A4 MXFP4 linear: activations rotated and quantized into the
 * workspace, then the FP4 GEMM with layer->bias.  w_codes / w_scales from
 * paro_mxfp4_quantize_weight; layer->qweight/qzeros/scales are not used. */
int paro_mxfp4_linear(const paro_w4_layer *layer, const uint8_t *w_codes, const uint8_t *w_scales, const void *x,
                      paro_dtype x_dt, int64_t tokens, void *y, paro_dtype y_dt, void *workspace,
                      size_t workspace_bytes, void *stream);
size_t paro_mxfp4_linear_workspace_bytes(const paro_w4_layer *layer, int64_t tokens);
/* The W4A4 MXFP4 linear with the layer's dense rotation prebuilt: hl from
 * paro_rotation_matrix for this layer and x_dt (I * 512 bytes, 16-byte
 * aligned, caller-owned, not written), as a model builds it once at load
 * time (it depends on the layer alone).  Results equal paro_mxfp4_linear's
 * bit for bit.  workspace: paro_mxfp4_linear_prepared_workspace_bytes(layer,
 * tokens) bytes (the activation codes and scales; no room for the rotation
 * matrix), 16-byte aligned, not overlapping x, y or hl.  Errors as
 * paro_mxfp4_linear, plus PARO_ERR_NULL for hl, PARO_ERR_ALIGN for its
 * alignment and PARO_ERR_SHAPE for its overlaps.  ("ParoQuant" blog, Bits
 * and formats: the MXFP4 variant of the W4A4 extension.) */
int paro_mxfp4_linear_prepared(const paro_w4_layer *layer, const void *hl, const uint8_t *w_codes,
                               const uint8_t *w_scales, const void *x, paro_dtype x_dt, int64_t tokens, void *y,
                               paro_dtype y_dt, void *workspace, size_t workspace_bytes, void *stream);
size_t paro_mxfp4_linear_prepared_workspace_bytes(const paro_w4_layer *layer, int64_t tokens);

/* Bytes of workspace the linear needs for this shape and path (0 allowed). */
size_t paro_w4a16_linear_workspace_bytes(const paro_w4_layer *layer, int64_t tokens,
                                         paro_dtype x_dt, paro_path path);

/* The path paro_w4a16_linear would take for this shape (never AUTO). */
paro_path paro_w4a16_linear_choose_path(const paro_w4_layer *layer, int64_t tokens);

/*
 * Host-side validation of a layer whose tensor pointers are HOST copies:
 * shape rules (G even and dividing I, O % 8 == 0, krot >= 1) and that every
 * pairs[t][g*G : (g+1)*G] is a permutation of 0..G-1.  Returns PARO_OK,
 * PARO_ERR_SHAPE, PARO_ERR_NULL or PARO_ERR_PAIRS.  Reads no device memory.
 */
int paro_validate_layer(const paro_w4_layer *host_layer);

/* Message for the last error on the calling thread ("" if none). */
const char *paro_last_error(void);

/* PARO_ABI_VERSION of the loaded library. */
int paro_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PARO_H */

/*
 * paro_ref.h - C-ABI of the fp64 CPU oracle (test infrastructure).
 *
 * This library is the checker for the GPU path declared in paro.h.  It is a
 * plain, slow, obviously correct host implementation of the rotated W4A16
 * linear and shares no code, header or constant with the GPU library.  Only
 * tests, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * What it computes (row-vector convention, all arithmetic in fp64):
 *
 *   Y = (X . D^-1 . R) . W_deq + b
 *
 *   - X            : tokens x I activations (fp16, bf16, fp32 or fp64 values)
 *   - D^-1         : the stored per-input-channel scales, multiplied in
 *                    ("ParoQuant" GPTQModel wiki, Concepts / Activation and
 *                    weight transforms: the saved channel_scales are D^-1)
 *   - R            : krot stages of disjoint Givens pair rotations, local to
 *                    each group of G input channels, applied in stage order
 *                    ("ParoQuant" wiki, Concepts / Pairwise Givens rotations)
 *   - W_deq[k][n]  : (q[k][n] - z[k/G][n]) * s[k/G][n], the affine dequant of
 *                    the AWQ-packed 4-bit codes ("GPTQ, GPTAQ, and RTN" wiki,
 *                    quantizer parameter selection; "ParoQuant" wiki, Triton
 *                    plans and tuning: subtract zero points, then multiply by
 *                    the group scales)
 *   - b            : optional fp16 bias.
 *
 * Stored-tensor shapes follow the "ParoQuant" wiki, Checkpoint and inference
 * implementation / Stored tensors.  Readings of points the pages leave open:
 *   - pairs[t][g*G + 2p], pairs[t][g*G + 2p + 1] are the local indices (a, b)
 *     of pair p of group g at stage t; theta[t][g*G/2 + p] is its angle.
 *   - AWQ nibble order: bits 4s..4s+3 of a packed word hold column 8w+ORD[s]
 *     with ORD = (0,2,4,6,1,3,5,7); equivalently column 8w+j sits at slot
 *     INV[j] with INV = (0,4,1,5,2,6,3,7).  Shifts are logical.
 *
 * Conventions: all pointers are HOST pointers owned by the caller; nothing is
 * retained after a call returns.  Functions return 0 on success and a
 * nonzero PARO_REF_ERR_* code on bad arguments (no partial output promised).
 * n_threads <= 0 means "all available OpenMP threads".
 */
#ifndef PARO_REF_H
#define PARO_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PARO_REF_F16 = 0,  /* IEEE binary16 bit patterns (uint16) */
  PARO_REF_BF16 = 1, /* bfloat16 bit patterns (uint16)      */
  PARO_REF_F32 = 2,  /* IEEE binary32 (float)               */
  PARO_REF_F64 = 3   /* IEEE binary64 (double), for exact test inputs */
};

enum {
  PARO_REF_OK = 0,
  PARO_REF_ERR_NULL = 1,         /* a required pointer is NULL              */
  PARO_REF_ERR_SHAPE = 2,        /* I, O, G, krot or tokens out of range    */
  PARO_REF_ERR_DTYPE = 3,        /* unknown dtype code                      */
  PARO_REF_ERR_PAIRS = 4,        /* a stage's group slice is no permutation */
  PARO_REF_ERR_CHECK_FAILED = 5, /* candidate outside the tolerance         */
  PARO_REF_ERR_NOMEM = 6         /* host allocation failed                  */
};

/* One rotated W4 linear layer, host copies of the stored tensors. */
typedef struct {
  int64_t in_features;     /* I                                            */
  int64_t out_features;    /* O, a multiple of 8                           */
  int32_t group_size;      /* G: even, divides I; -1 means G = I           */
  int32_t krot;            /* number of rotation stages, >= 1              */
  const int16_t *pairs;    /* [krot][I]   local pair indices               */
  const float *theta;      /* [krot][I/2] angles in radians                */
  const float *channel_scales; /* [I]     D^-1, multiplied in              */
  const int32_t *qweight;  /* [I][O/8]    AWQ-packed codes                 */
  const int32_t *qzeros;   /* [I/G][O/8]  AWQ-packed zero points           */
  const uint16_t *scales;  /* [I/G][O]    fp16 group scales                */
  const uint16_t *bias;    /* [O] fp16, or NULL for no bias                */
} paro_ref_layer;

/* Decode one fp16 / bf16 bit pattern to double (exact). */
double paro_ref_f16_to_double(uint16_t h);
double paro_ref_bf16_to_double(uint16_t h);

/* Round a double to the nearest fp16 / bf16 (ties to even); returns bits.
 * Overflow gives +-inf, NaN gives a quiet NaN. */
uint16_t paro_ref_round_f16(double v);
uint16_t paro_ref_round_bf16(double v);

/* Elementwise paro_ref_round_f16 (dt = PARO_REF_F16) or paro_ref_round_bf16
 * (dt = PARO_REF_BF16) of n doubles into out. */
int paro_ref_round_array(const double *v, int64_t n, int dt, uint16_t *out);

/* Check that every stage/group slice of pairs is a permutation of 0..G-1.
 * Returns PARO_REF_OK or PARO_REF_ERR_PAIRS. */
int paro_ref_check_pairs(const paro_ref_layer *layer);

/* x_r[m][k] = ((x . D^-1) . R)[m][k] for m < tokens, as double [tokens][I]. */
int paro_ref_scale_rotate(const paro_ref_layer *layer, const void *x, int x_dt,
                          int64_t tokens, double *x_r, int n_threads);

/* Unpack the codes: q_out [I][O] and/or z_out [I/G][O] (either may be NULL). */
int paro_ref_unpack(const paro_ref_layer *layer, uint8_t *q_out, uint8_t *z_out);

/* W_deq as double [I][O]. */
int paro_ref_dequant(const paro_ref_layer *layer, double *w_out, int n_threads);

/*
 * Backward of the scaling and rotation for a loss L with dL/dx_r = g (double
 * [tokens][I]), the calibration step of the method ("ParoQuant" wiki,
 * Straight-through estimation: optimization updates weights, angles and
 * channel scales; the pair formula of Concepts / Pairwise Givens rotations,
 * differentiated by the chain rule):
 *   gx     : double [tokens][I], dL/dx
 *   gtheta : double [krot][I/2], dL/dtheta summed over the tokens
 *   gcs    : double [I], dL/d(channel_scales) summed over the tokens
 * The forward states are kept row by row and walked back in stage order.
 */
int paro_ref_scale_rotate_backward(const paro_ref_layer *layer, const void *x, int x_dt, const double *g,
                                   int64_t tokens, double *gx, double *gtheta, double *gcs, int n_threads);
/*
 * Offline side of the method (the step before the stored tensors exist):
 *
 * W_r = W . D . R row by row ("ParoQuant" wiki, Concepts / Activation and
 * weight transforms; W is (out_features, in_features) = [O][I], the stored
 * channel_scales are D^-1, so they divide W's input channels).  Uses the
 * layer's I, O, G, krot, pairs, theta, channel_scales; w_r is double [O][I].
 */
int paro_ref_transform_weight(const paro_ref_layer *layer, const void *w, int w_dt, double *w_r,
                              int n_threads);
/*
 * Group round-to-nearest quantization of w_r (double [O][I]), per output row
 * n and group g of G input channels ("GPTQ, GPTAQ, and RTN" wiki, quantizer:
 * q = clamp(round(x / scale) + zero, 0, maxq), x_hat = scale (q - zero),
 * the observed range includes zero, symmetric ranges are +-max|x| with the
 * midpoint zero, affine zeros are round(-xmin / scale), all-zero ranges get a
 * finite sentinel range; "ParoQuant" wiki: four-bit codes, scales bounded to
 * [1e-5, 1e5], symmetric codes -8..7 exported with zero point 8).  maxq = 15,
 * rounding half to even, all decisions in double precision.
 *   q_out     : uint8 [I][O] codes 0..15 (the layout paro_ref_unpack returns)
 *   z_out     : uint8 [I/G][O] zero points
 *   s_out     : fp16 bits [I/G][O], the scale rounded to nearest even
 *   scale_out : double [I/G][O] unrounded scales, or NULL
 */
int paro_ref_quantize(int64_t O, int64_t I, int32_t group_size, const double *w_r, int sym,
                      uint8_t *q_out, uint8_t *z_out, uint16_t *s_out, double *scale_out);
/* AWQ pack of q [I][O] and z [I/G][O] into qweight [I][O/8] and qzeros
 * [I/G][O/8], the inverse of paro_ref_unpack (O % 8 == 0). */
int paro_ref_pack(int64_t I, int64_t O, int32_t group_size, const uint8_t *q, const uint8_t *z,
                  int32_t *qweight, int32_t *qzeros);
/*
 * MXFP4 (the four-bit-activation extension; "ParoQuant" blog, Bits and
 * formats).  Blocks of 32 consecutive elements of a row share an E8M0 scale
 * 2^(b - 127): b = floor(log2(max |v|)) - 2 + 127 clamped to 0..254 (0 for an
 * all-zero block); elements are E2M1 codes (bit 3 sign; magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6) of v / 2^(b - 127), nearest with ties to the even code,
 * clamped at 6, zero stored as +0.
 *   v: double [rows][K], K % 32 == 0
 *   codes: [rows][K/2] bytes, element 2j in the low nibble of byte j
 *   scales: [rows][K/32] biased exponents
 */
int paro_ref_mxfp4_quantize(int64_t rows, int64_t K, const double *v, uint8_t *codes, uint8_t *scales);
/* The values the codes and scales stand for, double [rows][K] (b = 255: NaN). */
int paro_ref_mxfp4_dequant(int64_t rows, int64_t K, const uint8_t *codes, const uint8_t *scales, double *out);
double paro_ref_e2m1_to_double(int code);
/* Y as double [tokens][O]. */
int paro_ref_linear(const paro_ref_layer *layer, const void *x, int x_dt,
                    int64_t tokens, double *y_out, int n_threads);

/*
 * Compute Y_ref (into y_ref_out when not NULL) and, when y is not NULL,
 * compare a candidate output y (y_dt bit patterns, [tokens][O]) with it:
 *   max_abs_err = max |y - Y_ref|,   max_abs_ref = max |Y_ref|.
 * Returns PARO_REF_OK when max_abs_err <= rel_tol * max_abs_ref (or when y is
 * NULL), PARO_REF_ERR_CHECK_FAILED otherwise; a NaN in y always fails.
 */
int paro_linear_ref_check(const paro_ref_layer *layer, const void *x, int x_dt,
                          int64_t tokens, const void *y, int y_dt,
                          double *y_ref_out, double rel_tol, int n_threads,
                          double *max_abs_err, double *max_abs_ref);

/* Number of OpenMP threads a call with n_threads would use. */
int paro_ref_threads(int n_threads);

#ifdef __cplusplus
}
#endif

#endif /* PARO_REF_H */

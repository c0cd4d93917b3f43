/*
 * paro_ref.c - fp64 CPU oracle for the rotated W4A16 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load the
 * library built from it.  It shares no code with the GPU library and is kept
 * deliberately plain: no blocking, no fusion, no reordering beyond the
 * definition, so that a reader can check each step against the pages by eye.
 * Independent rows/columns are spread over OpenMP threads, which does not
 * change any arithmetic.
 *
 * Every step cites the passage it follows:
 *   [P1] "ParoQuant", GPTQModel wiki (GPT-QModel 7.7.0)
 *   [P4] "GPTQ, GPTAQ, and RTN", GPTQModel wiki
 * Readings of points the pages leave open are listed in paro_ref.h.
 *
 * Parity pins: every function here is pinned by the CPU tests (worked
 * examples under tests/golden/, closed forms, invariants, brute force and
 * library special cases); none is "parity unpinned".
 */
#include "paro_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary16; bfloat16 = the top half of binary32).  */
/* ------------------------------------------------------------------------ */

double paro_ref_f16_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f; /* biased exponent, bias 15 */
  const int f = h & 0x3ff;        /* 10 fraction bits         */
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^(1-15-10) */
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
  }
  return sign ? -v : v;
}

double paro_ref_bf16_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 7) & 0xff; /* biased exponent, bias 127 */
  const int f = h & 0x7f;        /* 7 fraction bits           */
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133); /* subnormal: f * 2^(1-127-7) */
  } else if (e == 255) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(128 + f), e - 134); /* (1 + f/2^7) * 2^(e-127) */
  }
  return sign ? -v : v;
}

/*
 * Round |a| (finite, >= 0) to a binary format with p significand bits and
 * minimum normal exponent emin, ties to even.  Returns the rounded magnitude;
 * the caller encodes it.  rint() rounds half to even in the default mode.
 */
static double round_to_format(double a, int p, int emin) {
  if (a == 0.0) return 0.0;
  int e2;
  frexp(a, &e2);            /* a = m * 2^e2, m in [0.5, 1) */
  int e = e2 - 1;           /* floor(log2 a)              */
  if (e < emin) e = emin;   /* subnormal range: fixed quantum */
  const double quantum = ldexp(1.0, e - (p - 1));
  return rint(a / quantum) * quantum; /* a/quantum is exact (power of 2) */
}

static uint16_t encode_format(int sign, double v, int p, int emin, int ebias) {
  /* v is a rounded finite magnitude representable in the format */
  uint32_t bits;
  if (v == 0.0) {
    bits = 0;
  } else {
    int e2;
    frexp(v, &e2);
    int e = e2 - 1;
    if (e < emin) { /* subnormal: fraction = v / 2^(emin-(p-1)) */
      bits = (uint32_t)ldexp(v, -(emin - (p - 1)));
    } else {
      const uint32_t frac = (uint32_t)(ldexp(v, -(e - (p - 1))) - ldexp(1.0, p - 1));
      bits = ((uint32_t)(e + ebias) << (p - 1)) | frac;
    }
  }
  return (uint16_t)(((uint32_t)sign << 15) | bits);
}

uint16_t paro_ref_round_f16(double v) {
  if (isnan(v)) return 0x7e00;
  const int sign = signbit(v) ? 1 : 0;
  const double a = fabs(v);
  /* halfway between the largest finite 65504 and 2^16 rounds up (65504 is odd) */
  if (a >= 65520.0) return (uint16_t)((sign << 15) | 0x7c00);
  const double r = round_to_format(a, 11, -14);
  if (r >= 65536.0) return (uint16_t)((sign << 15) | 0x7c00);
  return encode_format(sign, r, 11, -14, 15);
}

uint16_t paro_ref_round_bf16(double v) {
  if (isnan(v)) return 0x7fc0;
  const int sign = signbit(v) ? 1 : 0;
  const double a = fabs(v);
  const double overflow = ldexp(2.0 - ldexp(1.0, -8), 127); /* tie above max */
  if (a >= overflow) return (uint16_t)((sign << 15) | 0x7f80);
  const double r = round_to_format(a, 8, -126);
  if (r >= ldexp(1.0, 128)) return (uint16_t)((sign << 15) | 0x7f80);
  return encode_format(sign, r, 8, -126, 127);
}

int paro_ref_round_array(const double *v, int64_t n, int dt, uint16_t *out) {
  if (n < 0) return PARO_REF_ERR_SHAPE;
  if (n > 0 && (!v || !out)) return PARO_REF_ERR_NULL;
  if (dt != PARO_REF_F16 && dt != PARO_REF_BF16) return PARO_REF_ERR_DTYPE;
  for (int64_t e = 0; e < n; ++e)
    out[e] = dt == PARO_REF_F16 ? paro_ref_round_f16(v[e]) : paro_ref_round_bf16(v[e]);
  return PARO_REF_OK;
}

static double load_elem(const void *p, int dt, int64_t idx) {
  if (dt == PARO_REF_F16) return paro_ref_f16_to_double(((const uint16_t *)p)[idx]);
  if (dt == PARO_REF_BF16) return paro_ref_bf16_to_double(((const uint16_t *)p)[idx]);
  if (dt == PARO_REF_F64) return ((const double *)p)[idx];
  return (double)((const float *)p)[idx];
}

int paro_ref_threads(int n_threads) {
#ifdef _OPENMP
  return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
  (void)n_threads;
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Argument checks.                                                          */
/* ------------------------------------------------------------------------ */

static int64_t group_of(const paro_ref_layer *L) {
  /* [P1] Concepts / Pairwise Givens rotations: group_size -1 means the whole
   * input width. */
  return L->group_size == -1 ? L->in_features : (int64_t)L->group_size;
}

static int check_shape(const paro_ref_layer *L) {
  if (!L) return PARO_REF_ERR_NULL;
  const int64_t I = L->in_features, O = L->out_features, G = group_of(L);
  /* [P1] groups have even width and divide the input width; the AWQ packer
   * needs O divisible by 8 (Stored tensors). */
  if (I <= 0 || O <= 0 || O % 8 != 0) return PARO_REF_ERR_SHAPE;
  if (G <= 0 || G % 2 != 0 || I % G != 0) return PARO_REF_ERR_SHAPE;
  if (G > 32768) return PARO_REF_ERR_SHAPE; /* int16 local indices */
  if (L->krot < 1) return PARO_REF_ERR_SHAPE;
  return PARO_REF_OK;
}

int paro_ref_check_pairs(const paro_ref_layer *L) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!L->pairs) return PARO_REF_ERR_NULL;
  const int64_t I = L->in_features, G = group_of(L);
  unsigned char *seen = (unsigned char *)malloc((size_t)G);
  if (!seen) return PARO_REF_ERR_NOMEM;
  rc = PARO_REF_OK;
  for (int t = 0; t < L->krot && rc == PARO_REF_OK; ++t) {
    for (int64_t g = 0; g < I / G && rc == PARO_REF_OK; ++g) {
      memset(seen, 0, (size_t)G);
      for (int64_t e = 0; e < G; ++e) {
        const int v = L->pairs[(int64_t)t * I + g * G + e];
        if (v < 0 || v >= G || seen[v]) { rc = PARO_REF_ERR_PAIRS; break; }
        seen[v] = 1;
      }
    }
  }
  free(seen);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Channel scaling and the pairwise rotation.                                */
/* ------------------------------------------------------------------------ */

/* cos/sin of every angle, once (libm, double precision); NULL if out of memory */
static double *angle_table(const paro_ref_layer *L) {
  const int64_t I = L->in_features;
  const int64_t nang = (int64_t)L->krot * (I / 2);
  double *cs_tab = (double *)malloc(sizeof(double) * 2 * (size_t)(nang > 0 ? nang : 1));
  if (!cs_tab) return NULL;
  for (int64_t e = 0; e < nang; ++e) {
    const double th = (double)L->theta[e];
    cs_tab[2 * e] = cos(th);
    cs_tab[2 * e + 1] = sin(th);
  }
  return cs_tab;
}

/* Rotation of one row in place: [P1] Concepts / Pairwise Givens rotations.
 * Stages run in order t = 0..krot-1; within a stage each group's channels form
 * disjoint pairs with group-local indices, so pairs are independent.  For a
 * pair (a, b) with angle theta:
 *     a' =  a cos(theta) + b sin(theta)
 *     b' = -a sin(theta) + b cos(theta)                                      */
static void rotate_row(const paro_ref_layer *L, const double *cs_tab, double *row) {
  const int64_t I = L->in_features, G = group_of(L), ngroups = I / G;
  for (int t = 0; t < L->krot; ++t) {
    for (int64_t g = 0; g < ngroups; ++g) {
      for (int64_t p = 0; p < G / 2; ++p) {
        const int64_t i = g * G + L->pairs[(int64_t)t * I + g * G + 2 * p];
        const int64_t j = g * G + L->pairs[(int64_t)t * I + g * G + 2 * p + 1];
        const int64_t ang = (int64_t)t * (I / 2) + g * (G / 2) + p;
        const double c = cs_tab[2 * ang], s = cs_tab[2 * ang + 1];
        const double a = row[i], b = row[j];
        row[i] = a * c + b * s;
        row[j] = -a * s + b * c;
      }
    }
  }
}

int paro_ref_scale_rotate(const paro_ref_layer *L, const void *x, int x_dt,
                          int64_t tokens, double *x_r, int n_threads) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (x_dt < PARO_REF_F16 || x_dt > PARO_REF_F64) return PARO_REF_ERR_DTYPE;
  if (tokens < 0) return PARO_REF_ERR_SHAPE;
  if (tokens == 0) return PARO_REF_OK;
  if (!x || !x_r || !L->theta || !L->channel_scales) return PARO_REF_ERR_NULL;
  rc = paro_ref_check_pairs(L);
  if (rc) return rc;
  const int64_t I = L->in_features;
  double *cs_tab = angle_table(L);
  if (!cs_tab) return PARO_REF_ERR_NOMEM;

#pragma omp parallel for schedule(static) num_threads(paro_ref_threads(n_threads))
  for (int64_t m = 0; m < tokens; ++m) {
    double *row = x_r + m * I;
    /* Step 1, channel scaling: [P1] Concepts / Activation and weight
     * transforms.  X_r = X D^-1 R and the stored channel_scales ARE D^-1,
     * so they multiply the activations. */
    for (int64_t k = 0; k < I; ++k)
      row[k] = load_elem(x, x_dt, m * I + k) * (double)L->channel_scales[k];
    /* Step 2, the staged rotation */
    rotate_row(L, cs_tab, row);
  }
  free(cs_tab);
  return PARO_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* AWQ unpack and affine dequantization.                                     */
/* ------------------------------------------------------------------------ */

/* Column 8w+j of a packed word lives in bits 4*SLOT_OF_COL[j] .. +3. */
static const int SLOT_OF_COL[8] = {0, 4, 1, 5, 2, 6, 3, 7};

static int nibble(int32_t word, int64_t col) {
  return (int)(((uint32_t)word >> (4 * SLOT_OF_COL[col % 8])) & 0xfu);
}

int paro_ref_unpack(const paro_ref_layer *L, uint8_t *q_out, uint8_t *z_out) {
  int rc = check_shape(L);
  if (rc) return rc;
  const int64_t I = L->in_features, O = L->out_features, G = group_of(L);
  const int64_t W = O / 8;
  /* [P1] Stored tensors: qweight is (I, O/8) and qzeros (I/G, O/8), eight
   * four-bit values per int32 word. */
  if (q_out) {
    if (!L->qweight) return PARO_REF_ERR_NULL;
    for (int64_t k = 0; k < I; ++k)
      for (int64_t n = 0; n < O; ++n)
        q_out[k * O + n] = (uint8_t)nibble(L->qweight[k * W + n / 8], n);
  }
  if (z_out) {
    if (!L->qzeros) return PARO_REF_ERR_NULL;
    for (int64_t g = 0; g < I / G; ++g)
      for (int64_t n = 0; n < O; ++n)
        z_out[g * O + n] = (uint8_t)nibble(L->qzeros[g * W + n / 8], n);
  }
  return PARO_REF_OK;
}

int paro_ref_dequant(const paro_ref_layer *L, double *w_out, int n_threads) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!w_out || !L->qweight || !L->qzeros || !L->scales) return PARO_REF_ERR_NULL;
  const int64_t I = L->in_features, O = L->out_features, G = group_of(L);
  const int64_t W = O / 8;
  /* [P4] affine quantizer: x_hat = scale * (q - zero); [P1] Triton plans:
   * the GEMM subtracts the zero points, then multiplies by the group scales.
   * (q - z) * s is exact in double. */
#pragma omp parallel for schedule(static) num_threads(paro_ref_threads(n_threads))
  for (int64_t k = 0; k < I; ++k) {
    const int64_t g = k / G;
    for (int64_t n = 0; n < O; ++n) {
      const int q = nibble(L->qweight[k * W + n / 8], n);
      const int z = nibble(L->qzeros[g * W + n / 8], n);
      const double s = paro_ref_f16_to_double(L->scales[g * O + n]);
      w_out[k * O + n] = (double)(q - z) * s;
    }
  }
  return PARO_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward of the channel scaling and rotation (the calibration step).       */
/* ------------------------------------------------------------------------ */

int paro_ref_scale_rotate_backward(const paro_ref_layer *L, const void *x, int x_dt, const double *g,
                                   int64_t tokens, double *gx, double *gtheta, double *gcs, int n_threads) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (x_dt < PARO_REF_F16 || x_dt > PARO_REF_F64) return PARO_REF_ERR_DTYPE;
  if (tokens < 0) return PARO_REF_ERR_SHAPE;
  if (!x || !g || !gx || !gtheta || !gcs || !L->theta || !L->channel_scales) return PARO_REF_ERR_NULL;
  rc = paro_ref_check_pairs(L);
  if (rc) return rc;
  const int64_t I = L->in_features, G = group_of(L), ngroups = I / G;
  const int krot = L->krot;
  const int64_t nang = (int64_t)krot * (I / 2);
  for (int64_t e = 0; e < nang; ++e) gtheta[e] = 0.0;
  for (int64_t k = 0; k < I; ++k) gcs[k] = 0.0;
  if (tokens == 0) return PARO_REF_OK;
  double *cs_tab = angle_table(L);
  if (!cs_tab) return PARO_REF_ERR_NOMEM;
  int nt = paro_ref_threads(n_threads);
  /* per-thread accumulators, summed in thread order afterwards */
  double *acc = (double *)calloc((size_t)nt * (size_t)(nang + I), sizeof(double));
  if (!acc) {
    free(cs_tab);
    return PARO_REF_ERR_NOMEM;
  }
  /* per-thread work rows, allocated before the parallel region so that every
   * thread reaches the worksharing loop below */
  double *work = (double *)malloc(sizeof(double) * (size_t)nt * (size_t)(krot + 2) * (size_t)I);
  if (!work) {
    free(acc);
    free(cs_tab);
    return PARO_REF_ERR_NOMEM;
  }
#pragma omp parallel num_threads(nt)
  {
#ifdef _OPENMP
    const int tid = omp_get_thread_num();
#else
    const int tid = 0;
#endif
    double *gth = acc + (size_t)tid * (size_t)(nang + I), *gc = gth + nang;
    /* states[t][k]: the row before stage t (states[krot] = x_r) */
    double *states = work + (size_t)tid * (size_t)(krot + 2) * (size_t)I;
    double *grad = states + (size_t)(krot + 1) * (size_t)I;
#pragma omp for schedule(static)
    for (int64_t m = 0; m < tokens; ++m) {
      /* forward, keeping every intermediate row: x_s = x * cs, then the
       * stages in order ([P1] Concepts / Pairwise Givens rotations) */
      for (int64_t k = 0; k < I; ++k)
        states[k] = load_elem(x, x_dt, m * I + k) * (double)L->channel_scales[k];
      for (int t = 0; t < krot; ++t) {
        double *in = states + (size_t)t * I, *out = states + (size_t)(t + 1) * I;
        for (int64_t k = 0; k < I; ++k) out[k] = in[k];
        for (int64_t gi = 0; gi < ngroups; ++gi)
          for (int64_t p = 0; p < G / 2; ++p) {
            const int64_t i = gi * G + L->pairs[(int64_t)t * I + gi * G + 2 * p];
            const int64_t j = gi * G + L->pairs[(int64_t)t * I + gi * G + 2 * p + 1];
            const int64_t ang = (int64_t)t * (I / 2) + gi * (G / 2) + p;
            const double c = cs_tab[2 * ang], sn = cs_tab[2 * ang + 1];
            out[i] = in[i] * c + in[j] * sn;
            out[j] = -in[i] * sn + in[j] * c;
          }
      }
      /* backward, stages in reverse: the chain rule through
       *   a' = a c + b s,  b' = -a s + b c
       * gives  dL/da = ga' c - gb' s,  dL/db = ga' s + gb' c  and, with
       * d a'/d theta = -a s + b c = b', d b'/d theta = -a c - b s = -a',
       *   dL/dtheta = ga' b' - gb' a'                                    */
      for (int64_t k = 0; k < I; ++k) grad[k] = g[m * I + k];
      for (int t = krot - 1; t >= 0; --t) {
        const double *out = states + (size_t)(t + 1) * I;
        for (int64_t gi = 0; gi < ngroups; ++gi)
          for (int64_t p = 0; p < G / 2; ++p) {
            const int64_t i = gi * G + L->pairs[(int64_t)t * I + gi * G + 2 * p];
            const int64_t j = gi * G + L->pairs[(int64_t)t * I + gi * G + 2 * p + 1];
            const int64_t ang = (int64_t)t * (I / 2) + gi * (G / 2) + p;
            const double c = cs_tab[2 * ang], sn = cs_tab[2 * ang + 1];
            const double ga = grad[i], gb = grad[j];
            gth[ang] += ga * out[j] - gb * out[i];
            grad[i] = ga * c - gb * sn;
            grad[j] = ga * sn + gb * c;
          }
      }
      /* channel scaling x_s = x * cs: dL/dx = dL/dx_s * cs, dL/dcs = dL/dx_s * x */
      for (int64_t k = 0; k < I; ++k) {
        const double xk = load_elem(x, x_dt, m * I + k);
        gx[m * I + k] = grad[k] * (double)L->channel_scales[k];
        gc[k] += grad[k] * xk;
      }
    }
  }
  free(work);
  for (int tid = 0; tid < nt; ++tid) {
    const double *gth = acc + (size_t)tid * (size_t)(nang + I), *gc = gth + nang;
    for (int64_t e = 0; e < nang; ++e) gtheta[e] += gth[e];
    for (int64_t k = 0; k < I; ++k) gcs[k] += gc[k];
  }
  free(acc);
  free(cs_tab);
  return PARO_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Offline transform, group quantization and AWQ packing of a dense weight.  */
/* ------------------------------------------------------------------------ */

int paro_ref_transform_weight(const paro_ref_layer *L, const void *w, int w_dt, double *w_r, int n_threads) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (w_dt < PARO_REF_F16 || w_dt > PARO_REF_F64) return PARO_REF_ERR_DTYPE;
  if (!w || !w_r || !L->theta || !L->channel_scales) return PARO_REF_ERR_NULL;
  rc = paro_ref_check_pairs(L);
  if (rc) return rc;
  const int64_t I = L->in_features, O = L->out_features;
  double *cs_tab = angle_table(L);
  if (!cs_tab) return PARO_REF_ERR_NOMEM;

#pragma omp parallel for schedule(static) num_threads(paro_ref_threads(n_threads))
  for (int64_t n = 0; n < O; ++n) {
    double *row = w_r + n * I;
    /* [P1] Concepts / Activation and weight transforms: W_r = W D R for W in
     * (out_features, in_features) order.  The stored channel_scales are D^-1,
     * so they divide the weight's input channels (the activations are
     * multiplied by them; the product X_r W_r^T is X W^T). */
    for (int64_t k = 0; k < I; ++k) row[k] = load_elem(w, w_dt, n * I + k) / (double)L->channel_scales[k];
    rotate_row(L, cs_tab, row);
  }
  free(cs_tab);
  return PARO_REF_OK;
}

int paro_ref_quantize(int64_t O, int64_t I, int32_t group_size, const double *w_r, int sym,
                      uint8_t *q_out, uint8_t *z_out, uint16_t *s_out, double *scale_out) {
  if (O <= 0 || I <= 0) return PARO_REF_ERR_SHAPE;
  const int64_t G = group_size == -1 ? I : group_size;
  if (G <= 0 || I % G != 0) return PARO_REF_ERR_SHAPE;
  if (!w_r || !q_out || !z_out || !s_out) return PARO_REF_ERR_NULL;
  const double maxq = 15.0;  /* four bits */
  for (int64_t n = 0; n < O; ++n) {
    for (int64_t g = 0; g < I / G; ++g) {
      const double *x = w_r + n * I + g * G;
      /* [P4] quantizer parameter selection: the observed range includes zero */
      double xmin = 0.0, xmax = 0.0;
      for (int64_t e = 0; e < G; ++e) {
        if (x[e] < xmin) xmin = x[e];
        if (x[e] > xmax) xmax = x[e];
      }
      /* symmetric: the range is widened to +-max|x| where it reaches below zero */
      if (sym) {
        if (-xmin > xmax) xmax = -xmin;
        if (xmin < 0.0) xmin = -xmax;
      }
      /* all-zero range: finite sentinel range */
      if (xmin == 0.0 && xmax == 0.0) {
        xmin = -1.0;
        xmax = 1.0;
      }
      double scale = (xmax - xmin) / maxq;
      /* [P1] quantizer scales are bounded to [1e-5, 1e5] */
      if (scale < 1e-5) scale = 1e-5;
      if (scale > 1e5) scale = 1e5;
      /* midpoint zero for symmetric, rounded -xmin/scale for affine (ties to even) */
      double zero = sym ? (maxq + 1.0) / 2.0 : rint(-xmin / scale);
      if (zero < 0.0) zero = 0.0;
      if (zero > maxq) zero = maxq;
      z_out[g * O + n] = (uint8_t)zero;
      s_out[g * O + n] = paro_ref_round_f16(scale);
      if (scale_out) scale_out[g * O + n] = scale;
      /* [P4] q = clamp(round(x / scale) + zero, 0, maxq), round half to even */
      for (int64_t e = 0; e < G; ++e) {
        double q = rint(x[e] / scale) + zero;
        if (q < 0.0) q = 0.0;
        if (q > maxq) q = maxq;
        q_out[(g * G + e) * O + n] = (uint8_t)q;
      }
    }
  }
  return PARO_REF_OK;
}

int paro_ref_pack(int64_t I, int64_t O, int32_t group_size, const uint8_t *q, const uint8_t *z,
                  int32_t *qweight, int32_t *qzeros) {
  if (O <= 0 || I <= 0 || O % 8 != 0) return PARO_REF_ERR_SHAPE;
  const int64_t G = group_size == -1 ? I : group_size;
  if (G <= 0 || I % G != 0) return PARO_REF_ERR_SHAPE;
  if (!q || !z || !qweight || !qzeros) return PARO_REF_ERR_NULL;
  /* [P1] Stored tensors: AWQ layout, 8 columns per int32 word; column 8w+j
   * goes to bits 4*SLOT_OF_COL[j] (the order paro_ref_unpack reads). */
  for (int64_t k = 0; k < I; ++k)
    for (int64_t w = 0; w < O / 8; ++w) {
      uint32_t word = 0;
      for (int j = 0; j < 8; ++j) word |= (uint32_t)(q[k * O + 8 * w + j] & 0xfu) << (4 * SLOT_OF_COL[j]);
      qweight[k * (O / 8) + w] = (int32_t)word;
    }
  for (int64_t g = 0; g < I / G; ++g)
    for (int64_t w = 0; w < O / 8; ++w) {
      uint32_t word = 0;
      for (int j = 0; j < 8; ++j) word |= (uint32_t)(z[g * O + 8 * w + j] & 0xfu) << (4 * SLOT_OF_COL[j]);
      qzeros[g * (O / 8) + w] = (int32_t)word;
    }
  return PARO_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* MXFP4, the four-bit-activation extension ("ParoQuant" blog, Bits and       */
/* formats: W4A4 with an MXFP4 variant).  OCP microscaling format: each block */
/* of 32 consecutive elements along a row shares one E8M0 scale, a power of   */
/* two 2^(b - 127) with b = 0..254; each element is E2M1 (sign, two exponent  */
/* bits, one mantissa bit) with magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The   */
/* block exponent is floor(log2(max |v|)) minus 2, the exponent of E2M1's     */
/* largest value (6 = 1.5 * 2^2); elements are v / 2^exp rounded to the       */
/* nearest E2M1 value, ties to the even code, clamped at 6.                    */
/* ------------------------------------------------------------------------ */

static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double paro_ref_e2m1_to_double(int code) {
  return (code & 8 ? -1.0 : 1.0) * E2M1_MAG[code & 7];
}

/* Nearest magnitude code of a >= 0, ties to the even code (brute force). */
static int e2m1_nearest(double a) {
  int best = 0;
  double bd = fabs(a - E2M1_MAG[0]);
  for (int c = 1; c < 8; ++c) {
    const double d = fabs(a - E2M1_MAG[c]);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bd = d;
    }
  }
  return best;
}

int paro_ref_mxfp4_quantize(int64_t rows, int64_t K, const double *v, uint8_t *codes, uint8_t *scales) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return PARO_REF_ERR_SHAPE;
  if (rows > 0 && (!v || !codes || !scales)) return PARO_REF_ERR_NULL;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < K / 32; ++b) {
      const double *blk = v + r * K + 32 * b;
      double amax = 0.0;
      for (int e = 0; e < 32; ++e) amax = fmax(amax, fabs(blk[e]));
      int biased = 0; /* an all-zero block: the smallest scale, all codes 0 */
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* amax = f * 2^ex, 0.5 <= f < 1: floor(log2 amax) = ex - 1 */
        biased = (ex - 1) - 2 + 127;
        if (biased < 0) biased = 0;
        if (biased > 254) biased = 254;
      }
      scales[r * (K / 32) + b] = (uint8_t)biased;
      const double X = ldexp(1.0, biased - 127);
      for (int e = 0; e < 32; e += 2) {
        int c[2];
        for (int h = 0; h < 2; ++h) {
          const double q = blk[e + h] / X;
          const int m = e2m1_nearest(fabs(q));
          c[h] = (q < 0.0 && m != 0) ? (m | 8) : m; /* zero is stored as +0 */
        }
        /* element 2j in the low nibble of byte j, 2j+1 in the high nibble */
        codes[r * (K / 2) + 16 * b + e / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  return PARO_REF_OK;
}

int paro_ref_mxfp4_dequant(int64_t rows, int64_t K, const uint8_t *codes, const uint8_t *scales, double *out) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return PARO_REF_ERR_SHAPE;
  if (rows > 0 && (!codes || !scales || !out)) return PARO_REF_ERR_NULL;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const int byte = codes[r * (K / 2) + k / 2];
      const int c = (k & 1) ? (byte >> 4) : (byte & 15);
      const int biased = scales[r * (K / 32) + k / 32];
      out[r * K + k] = biased == 255 ? NAN : paro_ref_e2m1_to_double(c) * ldexp(1.0, biased - 127);
    }
  return PARO_REF_OK;
}

/* ------------------------------------------------------------------------ */
/* The linear: Y = X_r . W_deq + b.                                          */
/* ------------------------------------------------------------------------ */

int paro_ref_linear(const paro_ref_layer *L, const void *x, int x_dt,
                    int64_t tokens, double *y_out, int n_threads) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (tokens < 0) return PARO_REF_ERR_SHAPE;
  if (tokens == 0) return PARO_REF_OK;
  if (!y_out) return PARO_REF_ERR_NULL;
  const int64_t I = L->in_features, O = L->out_features;

  double *xr = (double *)malloc(sizeof(double) * (size_t)(tokens * I));
  double *w = (double *)malloc(sizeof(double) * (size_t)(I * O));
  if (!xr || !w) { free(xr); free(w); return PARO_REF_ERR_NOMEM; }
  rc = paro_ref_scale_rotate(L, x, x_dt, tokens, xr, n_threads);
  if (!rc) rc = paro_ref_dequant(L, w, n_threads);
  if (rc) { free(xr); free(w); return rc; }

  /* [P1] Concepts / Activation and weight transforms: the replayed linear is
   * Y = X_r Q(W_r)^T + b; W_deq[k][n] is Q(W_r)^T in (I, O) layout.  Each
   * output element is a plain sum over k; columns are split into chunks only
   * to spread independent outputs over threads. */
  enum { CHUNK = 256 };
  const int64_t nchunks = (O + CHUNK - 1) / CHUNK;
#pragma omp parallel for collapse(2) schedule(static) num_threads(paro_ref_threads(n_threads))
  for (int64_t m = 0; m < tokens; ++m) {
    for (int64_t c = 0; c < nchunks; ++c) {
      double acc[CHUNK];
      const int64_t n0 = c * CHUNK;
      const int64_t nn = (O - n0) < CHUNK ? (O - n0) : CHUNK;
      for (int64_t n = 0; n < nn; ++n) acc[n] = 0.0;
      for (int64_t k = 0; k < I; ++k) {
        const double xv = xr[m * I + k];
        const double *wrow = w + k * O + n0;
        for (int64_t n = 0; n < nn; ++n) acc[n] += xv * wrow[n];
      }
      for (int64_t n = 0; n < nn; ++n) {
        const double b = L->bias ? paro_ref_f16_to_double(L->bias[n0 + n]) : 0.0;
        y_out[m * O + n0 + n] = acc[n] + b;
      }
    }
  }
  free(xr);
  free(w);
  return PARO_REF_OK;
}

int paro_linear_ref_check(const paro_ref_layer *L, const void *x, int x_dt,
                          int64_t tokens, const void *y, int y_dt,
                          double *y_ref_out, double rel_tol, int n_threads,
                          double *max_abs_err, double *max_abs_ref) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (y && (y_dt < PARO_REF_F16 || y_dt > PARO_REF_F64)) return PARO_REF_ERR_DTYPE;
  if (tokens < 0) return PARO_REF_ERR_SHAPE;
  const int64_t O = L->out_features;
  double *yref = y_ref_out;
  if (!yref && tokens > 0) {
    yref = (double *)malloc(sizeof(double) * (size_t)(tokens * O));
    if (!yref) return PARO_REF_ERR_NOMEM;
  }
  rc = paro_ref_linear(L, x, x_dt, tokens, yref, n_threads);
  double err = 0.0, ref = 0.0;
  int nan_seen = 0;
  if (!rc) {
    for (int64_t e = 0; e < tokens * O; ++e) {
      const double r = fabs(yref[e]);
      if (r > ref) ref = r;
      if (y) {
        const double v = load_elem(y, y_dt, e);
        if (isnan(v)) nan_seen = 1;
        const double d = fabs(v - yref[e]);
        if (d > err) err = d;
      }
    }
  }
  if (yref != y_ref_out) free(yref);
  if (rc) return rc;
  if (max_abs_err) *max_abs_err = nan_seen ? NAN : err;
  if (max_abs_ref) *max_abs_ref = ref;
  if (y && (nan_seen || !(err <= rel_tol * ref))) return PARO_REF_ERR_CHECK_FAILED;
  return PARO_REF_OK;
}

/*
 * psffn_oracle.c -- plain, slow, CPU reference for the predictor-gated sparse FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it follows:
 *   - "PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU" (Elamur
 *     Research summary), Summary, 2nd paragraph: small per-layer predictors guess which
 *     neurons of the MLP will fire, and neuron-level kernels compute only those and skip the
 *     rest.
 *   - same page, Interesting ideas, I4: those kernels work directly on the rows and columns
 *     of the weight matrices (no sparse-format conversion).
 *   - same page, Interesting ideas, I1 and Summary, 2nd paragraph: neurons are profiled
 *     offline by how often they fire; hot ones go to the fastest memory.
 *   - same page, Key points (sparsity): ReLU FFNs are very sparse, SwiGLU ones much less.
 *
 * So the sparse FFN is, by definition, the dense FFN restricted to the predicted neuron
 * set.  Every routine below is that definition written out as scalar loops over the STORED
 * bytes (fp32, fp16 or 4-bit groups decoded exactly), accumulating in fp64, with no
 * blocking, no reordering and no BLAS.  Where the pages leave a step open (predictor form,
 * threshold, 4-bit layout, layer norm in the stack) the reading used is stated at the
 * routine.
 *
 * Parity pins: every routine is pinned by tests in tests/test_oracle_*.py against closed
 * forms, invariants, library routines and hand-worked fixtures (tests/golden/).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* storage codes */
#define ORC_F32 0
#define ORC_F16 1
#define ORC_I4G128 2 /* weights only: 4-bit signed nibbles, one fp16 scale per 128 elements */

#define ORC_RELU 0
#define ORC_SWIGLU 1

/* IEEE 754 binary16 -> double, exactly (every half is representable in a double). */
double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* double -> binary16 with round-to-nearest-even (used only where the method stores a value
 * in fp16: the layer-norm output that feeds each FFN of the decode stack). */
uint16_t orc_double_to_half(double v) {
  uint16_t sign = (uint16_t)(signbit(v) ? 0x8000 : 0);
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(sign | 0x7e00);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00); /* rounds to infinity */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: quantum 2^-24 */
    double q = a * ldexp(1.0, 24);
    double r = nearbyint(q); /* default rounding mode is to-nearest-even */
    return (uint16_t)(sign | (uint16_t)r); /* r == 1024 becomes the smallest normal */
  }
  int e;
  double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  /* a = (1 + m/1024) * 2^(E), E = e - 1, quantum 2^(E-10) */
  int E = e - 1;
  double q = ldexp(a, 10 - E); /* in [1024, 2048) */
  double r = nearbyint(q);
  if (r >= 2048.0) {
    r = 1024.0;
    E += 1;
  }
  (void)f;
  if (E > 15) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024));
}

/* The value of every binary16 bit pattern, filled once from orc_half_to_double when the library
 * loads, so that reading an fp16 element is a lookup rather than a libm call. */
static double half_value[65536];

__attribute__((constructor)) static void fill_half_values(void) {
  for (int h = 0; h < 65536; ++h) half_value[h] = orc_half_to_double((uint16_t)h);
}

/* Element (row, col) of a dense row-major matrix with `ld` columns, stored as fp32 or fp16. */
static double dense_elem(int dt, const void* p, size_t ld, size_t row, size_t col) {
  size_t at = row * ld + col;
  if (dt == ORC_F32) return (double)((const float*)p)[at];
  return half_value[((const uint16_t*)p)[at]];
}

/* Element (row, col) of a 4-bit weight matrix with `d` columns.  Reading of the format
 * (the pages only say the models run 4-bit quantised, Summary, 1st paragraph, and Key points,
 * speed): each row holds d/2 bytes; element 2j sits in the low nibble of byte j and element
 * 2j+1 in the high nibble; a nibble is a two's-complement integer in [-8, 7]; the value is
 * that integer times the fp16 scale of its group of 128 consecutive elements of the row. */
double orc_i4_elem(const uint8_t* packed, const uint16_t* scales, size_t d, size_t row, size_t col) {
  uint8_t byte = packed[row * (d / 2) + col / 2];
  int nib = (col & 1) ? (byte >> 4) : (byte & 15);
  int q = nib >= 8 ? nib - 16 : nib;
  double s = half_value[scales[row * (d / 128) + col / 128]];
  return (double)q * s;
}

static double weight_elem(int dt, const void* w, const uint16_t* s, size_t d, size_t row, size_t col) {
  if (dt == ORC_I4G128) return orc_i4_elem((const uint8_t*)w, s, d, row, col);
  return dense_elem(dt, w, d, row, col);
}

/* Predictor (Summary, 2nd paragraph: a lightweight per-layer predictor).  Reading: a linear
 * low-rank map, h = A x (A is r x d) then logit l = Q h + c (Q is F x r).  Neuron i is
 * predicted to fire when sigmoid(l_i) > 1/2, i.e. l_i > 0; a general threshold is taken on
 * the logit.  logits[b*F + i] for token b of a batch of B. */
void orc_predict_logits(int dt_p, const void* A, const void* Q, const float* c, int d, int r, int F, int dt_x,
                        const void* x, int B, double* logits) {
  double* h = (double*)malloc(sizeof(double) * (size_t)r);
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < r; ++j) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += dense_elem(dt_p, A, d, j, k) * dense_elem(dt_x, x, d, b, k);
      h[j] = s;
    }
    for (int i = 0; i < F; ++i) {
      double s = (double)c[i];
      for (int j = 0; j < r; ++j) s += dense_elem(dt_p, Q, r, i, j) * h[j];
      logits[(size_t)b * F + i] = s;
    }
  }
  free(h);
}

/* "Skip the rest" (Summary, 2nd paragraph): the neurons kept are those whose logit exceeds
 * the threshold for at least one token of the batch (a batch shares one neuron set, the
 * union of the per-token sets).  Written in ascending neuron order.  Returns the count. */
int orc_compact(const double* logits, int B, int F, double thr, int32_t* idx) {
  int n = 0;
  for (int i = 0; i < F; ++i) {
    int on = 0;
    for (int b = 0; b < B; ++b)
      if (logits[(size_t)b * F + i] > thr) on = 1;
    if (on) idx[n++] = i;
  }
  return n;
}

/* Hot prefix (Elamur summary, Summary 1st paragraph: a small set of hot neurons fires for
 * almost every input; Interesting ideas, I1: place the most used parts first).  With the neurons
 * in hot-first order, the first n_hot of them are kept for every batch without consulting the
 * predictor; the predictor decides only for the rest (same rule as orc_compact).  Ascending
 * order; returns the count. */
int orc_compact_hot(const double* logits, int B, int F, double thr, int n_hot, int32_t* idx) {
  int n = 0;
  for (int i = 0; i < F; ++i) {
    int on = i < n_hot;
    for (int b = 0; b < B && !on; ++b)
      if (logits[(size_t)b * F + i] > thr) on = 1;
    if (on) idx[n++] = i;
  }
  return n;
}

/* Activation of neuron i for token b (Interesting ideas, I4: work on whole rows).
 *   ReLU  : a = max(W_up[i] . x + b_up[i], 0)
 *   SwiGLU: a = silu(W_gate[i] . x + b_gate[i]) * (W_up[i] . x + b_up[i]),  silu(g) = g / (1 + e^-g)
 * Null bias pointers mean zero bias. */
static double neuron_act(int dt_w, int act, int d, const void* w_up, const uint16_t* s_up, const void* w_gate,
                         const uint16_t* s_gate, const float* b_up, const float* b_gate, int dt_x, const void* x,
                         int b, int i) {
  double u = b_up ? (double)b_up[i] : 0.0;
  for (int k = 0; k < d; ++k) u += weight_elem(dt_w, w_up, s_up, d, i, k) * dense_elem(dt_x, x, d, b, k);
  if (act == ORC_RELU) return u > 0.0 ? u : 0.0;
  double g = b_gate ? (double)b_gate[i] : 0.0;
  for (int k = 0; k < d; ++k) g += weight_elem(dt_w, w_gate, s_gate, d, i, k) * dense_elem(dt_x, x, d, b, k);
  return g / (1.0 + exp(-g)) * u;
}

/* Activations of the listed neurons: a[k*B + b] for k < count. */
void orc_activations(int dt_w, int act, int d, const void* w_up, const uint16_t* s_up, const void* w_gate,
                     const uint16_t* s_gate, const float* b_up, const float* b_gate, int dt_x, const void* x, int B,
                     const int32_t* idx, int count, double* a) {
  for (int k = 0; k < count; ++k)
    for (int b = 0; b < B; ++b)
      a[(size_t)k * B + b] =
          neuron_act(dt_w, act, d, w_up, s_up, w_gate, s_gate, b_up, b_gate, dt_x, x, b, idx[k]);
}

/* Sparse FFN over a given neuron list: y_b = b_down + sum over listed neurons i of
 * a_i(x_b) * W_down^T[i], with W_down^T stored neuron-major (row i = column i of W_down).
 * The dense FFN is this with the list 0..F-1.  y[b*d + j]. */
void orc_sparse_ffn(int dt_w, int act, int d, int F, const void* w_up, const uint16_t* s_up, const void* w_gate,
                    const uint16_t* s_gate, const void* w_dT, const uint16_t* s_dT, const float* b_up,
                    const float* b_gate, const float* b_down, int dt_x, const void* x, int B, const int32_t* idx,
                    int count, double* y) {
  (void)F;
  double* a = (double*)malloc(sizeof(double) * ((size_t)count * B + 1));
  orc_activations(dt_w, act, d, w_up, s_up, w_gate, s_gate, b_up, b_gate, dt_x, x, B, idx, count, a);
  /* every y[b][j] starts at b_down[j] and takes the listed neurons' terms in list order; the terms
   * are added row by row (one W_down^T row at a time) so the rows are read in memory order */
  for (int b = 0; b < B; ++b) {
    double* yb = y + (size_t)b * d;
    for (int j = 0; j < d; ++j) yb[j] = b_down ? (double)b_down[j] : 0.0;
    for (int k = 0; k < count; ++k) {
      const double ak = a[(size_t)k * B + b];
      for (int j = 0; j < d; ++j) yb[j] += ak * weight_elem(dt_w, w_dT, s_dT, d, idx[k], j);
    }
  }
  free(a);
}

/* Offline activation profile (Summary, 2nd paragraph; Interesting ideas, I1): for each neuron,
 * the number of the T tokens for which it truly fires -- pre-activation > 0 for ReLU, gate
 * pre-activation > 0 for SwiGLU.  `thr` generalises the 0 (the definition is thr = 0; other
 * values bracket a count computed in lower precision). */
void orc_fire_counts(int dt_w, int act, int d, int F, const void* w_up, const uint16_t* s_up, const void* w_gate,
                     const uint16_t* s_gate, const float* b_up, const float* b_gate, int dt_x, const void* x, int T,
                     double thr, int32_t* counts) {
  const void* w = act == ORC_RELU ? w_up : w_gate;
  const uint16_t* s = act == ORC_RELU ? s_up : s_gate;
  const float* bias = act == ORC_RELU ? b_up : b_gate;
  for (int i = 0; i < F; ++i) {
    int n = 0;
    for (int t = 0; t < T; ++t) {
      double z = bias ? (double)bias[i] : 0.0;
      for (int k = 0; k < d; ++k) z += weight_elem(dt_w, w, s, d, i, k) * dense_elem(dt_x, x, d, t, k);
      if (z > thr) ++n;
    }
    counts[i] = n;
  }
}

/* The deciding pre-activations themselves: z[t][i] = the ReLU pre-activation W_up[i].x_t + b_up[i],
 * or for SwiGLU the gate W_gate[i].x_t + b_gate[i] (fp64, the stored weights decoded exactly) --
 * the quantity whose sign orc_fire_counts counts, for tests that need its distance from zero. */
void orc_pre_activations(int dt_w, int act, int d, int F, const void* w_up, const uint16_t* s_up, const void* w_gate,
                         const uint16_t* s_gate, const float* b_up, const float* b_gate, int dt_x, const void* x,
                         int T, double* z) {
  const void* w = act == ORC_RELU ? w_up : w_gate;
  const uint16_t* s = act == ORC_RELU ? s_up : s_gate;
  const float* bias = act == ORC_RELU ? b_up : b_gate;
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < F; ++i) {
      double v = bias ? (double)bias[i] : 0.0;
      for (int k = 0; k < d; ++k) v += weight_elem(dt_w, w, s, d, i, k) * dense_elem(dt_x, x, d, t, k);
      z[(size_t)t * F + i] = v;
    }
}

/* Hot-first order (Interesting ideas, I1: the most used parts go first / to the fastest
 * memory).  perm[k] = the neuron placed at position k: descending fire count, ties broken by
 * ascending original index (a stable order). */
static const int32_t* g_counts;
static int cmp_hot_first(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  if (g_counts[a] != g_counts[b]) return g_counts[a] > g_counts[b] ? -1 : 1;
  return a < b ? -1 : (a > b ? 1 : 0);
}
void orc_hot_first_perm(const int32_t* counts, int F, int32_t* perm) {
  for (int i = 0; i < F; ++i) perm[i] = i;
  g_counts = counts;
  qsort(perm, (size_t)F, sizeof(int32_t), cmp_hot_first);
  g_counts = NULL;
}

/* Layer norm of each token of the fp32 residual stream, gamma = 1, beta = 0, population
 * variance: out = (x - mean) / sqrt(var + eps).  Used only by the decode-stack glue. */
void orc_layernorm(const float* x, int B, int d, double eps, double* out) {
  for (int b = 0; b < B; ++b) {
    const float* xr = x + (size_t)b * d;
    double m = 0.0;
    for (int k = 0; k < d; ++k) m += (double)xr[k];
    m /= d;
    double v = 0.0;
    for (int k = 0; k < d; ++k) v += ((double)xr[k] - m) * ((double)xr[k] - m);
    v /= d;
    double inv = 1.0 / sqrt(v + eps);
    for (int k = 0; k < d; ++k) out[(size_t)b * d + k] = ((double)xr[k] - m) * inv;
  }
}

/*
 * End to end from a plain C11 caller on the GPU, with no Python and no torch: device memory from
 * hipMalloc, one psffn_layer call per batch size, results copied back and checked against the C
 * oracle (oracle/psffn_oracle.c, compiled into this test program; test infrastructure only).
 * Built and run by tests/test_c_consumer_gpu.py.  Prints one line per check and exits with the
 * number of failed checks.
 *
 * Layer: d 512, F 1024, r 64, fp16 predictor and fp16 ReLU weights, biases, seeded uniform
 * values (splitmix64), logit bias -0.2 so that about one neuron in six fires at one token.  Batch
 * 1 takes the streamed one-token pipeline, batch 4 the MFMA batch pipeline.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "psffn.h"

/* the C oracle (oracle/psffn_oracle.c) */
double orc_half_to_double(uint16_t h);
uint16_t orc_double_to_half(double v);
void orc_predict_logits(int dt_p, const void* A, const void* Q, const float* c, int d, int r, int F, int dt_x,
                        const void* x, int B, double* logits);
int orc_compact(const double* logits, int B, int F, double thr, int32_t* idx);
void orc_sparse_ffn(int dt_w, int act, int d, int F, const void* w_up, const uint16_t* s_up, const void* w_gate,
                    const uint16_t* s_gate, const void* w_dT, const uint16_t* s_dT, const float* b_up,
                    const float* b_gate, const float* b_down, int dt_x, const void* x, int B, const int32_t* idx,
                    int count, double* y);
#define ORC_F16 1
#define ORC_RELU 0

enum { D = 512, F = 1024, R = 64, MAXB = 4 };

static int failed = 0;
static void check(int ok, const char* what, int B) {
  printf("%s B=%d %s\n", ok ? "ok  " : "FAIL", B, what);
  if (!ok) ++failed;
}

static uint64_t rng_state = 0x5eed1234abcdull;
static double uniform(void) { /* splitmix64 -> [-1, 1) */
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) * 0x1.0p-52 - 1.0;
}
static void fill_half(uint16_t* p, size_t n, double scale) {
  for (size_t i = 0; i < n; ++i) p[i] = orc_double_to_half(scale * uniform());
}
static void fill_float(float* p, size_t n, double offset, double scale) {
  for (size_t i = 0; i < n; ++i) p[i] = (float)(offset + scale * uniform());
}

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));              \
      return 100;                                                         \
    }                                                                     \
  } while (0)

static void* dev_copy(const void* host, size_t bytes) {
  void* p = NULL;
  if (hipMalloc(&p, bytes) != hipSuccess) return NULL;
  if (hipMemcpy(p, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return p;
}

int main(void) {
  static uint16_t A[R * D], Q[F * R], w_up[F * D], w_dT[F * D], x[MAXB * D];
  static float c[F], b_up[F], b_down[D];
  fill_half(A, (size_t)R * D, 1.0 / sqrt((double)D));
  fill_half(Q, (size_t)F * R, 1.0 / sqrt((double)R));
  fill_float(c, F, -0.2, 0.05);
  fill_half(w_up, (size_t)F * D, 1.0 / sqrt((double)D));
  fill_half(w_dT, (size_t)F * D, 1.0 / sqrt((double)F));
  fill_float(b_up, F, 0.0, 0.1);
  fill_float(b_down, D, 0.0, 0.1);
  fill_half(x, (size_t)MAXB * D, 1.0);

  psffn_predictor P;
  memset(&P, 0, sizeof P);
  P.d = D;
  P.F = F;
  P.r = R;
  P.dt = PSFFN_F16;
  P.A = dev_copy(A, sizeof A);
  P.Q = dev_copy(Q, sizeof Q);
  P.c = (const float*)dev_copy(c, sizeof c);
  psffn_ffn W;
  memset(&W, 0, sizeof W);
  W.d = D;
  W.F = F;
  W.dt = PSFFN_F16;
  W.act = PSFFN_RELU;
  W.w_up = dev_copy(w_up, sizeof w_up);
  W.w_dT = dev_copy(w_dT, sizeof w_dT);
  W.b_up = (const float*)dev_copy(b_up, sizeof b_up);
  W.b_down = (const float*)dev_copy(b_down, sizeof b_down);
  void* dx = dev_copy(x, sizeof x);
  if (!P.A || !P.Q || !P.c || !W.w_up || !W.w_dT || !W.b_up || !W.b_down || !dx) {
    printf("FAIL device allocation or copy\n");
    return 100;
  }
  const size_t ws_bytes = psffn_workspace_bytes(&P, &W, MAXB);
  void *ws = NULL, *didx = NULL, *dcount = NULL, *dlogits = NULL, *dy = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc(&didx, sizeof(int32_t) * F));
  HIP_OK(hipMalloc(&dcount, sizeof(int32_t)));
  HIP_OK(hipMalloc(&dlogits, sizeof(float) * MAXB * F));
  HIP_OK(hipMalloc(&dy, sizeof(float) * MAXB * D));
  check(ws_bytes > 0 && psffn_workspace_init(ws, ws_bytes, NULL) == PSFFN_OK, "workspace sized and initialised", 0);

  static int32_t idx[F], idx_ref[F];
  static float logits[MAXB * F], y[MAXB * D];
  static double logits_ref[MAXB * F], y_ref[MAXB * D];
  const int batches[2] = {1, 4};
  for (int t = 0; t < 2; ++t) {
    const int B = batches[t];
    const psffn_status st = psffn_layer(&P, &W, dx, B, 0.0f, (int32_t*)didx, (int32_t*)dcount, (float*)dlogits,
                                        (float*)dy, 0, ws, ws_bytes, NULL);
    check(st == PSFFN_OK, "psffn_layer returns PSFFN_OK", B);
    HIP_OK(hipDeviceSynchronize());
    int32_t n = -1;
    HIP_OK(hipMemcpy(&n, dcount, sizeof n, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(idx, didx, sizeof(int32_t) * F, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(logits, dlogits, sizeof(float) * (size_t)B * F, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, dy, sizeof(float) * (size_t)B * D, hipMemcpyDeviceToHost));

    /* logits against the oracle's fp64 values */
    orc_predict_logits(ORC_F16, A, Q, c, D, R, F, ORC_F16, x, B, logits_ref);
    double lmax = 0.0, lerr = 0.0;
    for (int i = 0; i < B * F; ++i) {
      lmax = fmax(lmax, fabs(logits_ref[i]));
      lerr = fmax(lerr, fabs((double)logits[i] - logits_ref[i]));
    }
    check(lerr <= 1e-5 * (1.0 + lmax), "logits within 1e-5 of the oracle", B);

    /* the active set: ascending, and the oracle's except neurons within 1e-6 of the threshold */
    const int n_ref = orc_compact(logits_ref, B, F, 0.0, idx_ref);
    int ascending = n >= 0 && n <= F;
    for (int k = 1; ascending && k < n; ++k) ascending = idx[k] > idx[k - 1];
    check(ascending, "the list is strictly ascending", B);
    static char in_got[F], in_ref[F];
    memset(in_got, 0, sizeof in_got);
    memset(in_ref, 0, sizeof in_ref);
    for (int k = 0; ascending && k < n; ++k)
      if (idx[k] >= 0 && idx[k] < F) in_got[idx[k]] = 1;
    for (int k = 0; k < n_ref; ++k) in_ref[idx_ref[k]] = 1;
    int set_ok = ascending;
    for (int i = 0; i < F; ++i) {
      if (in_got[i] == in_ref[i]) continue;
      double m = -INFINITY;
      for (int b = 0; b < B; ++b) m = fmax(m, logits_ref[(size_t)b * F + i]);
      if (fabs(m) >= 1e-6) set_ok = 0;
    }
    check(set_ok && n > 0 && n < F, "the active set matches the oracle (outside the 1e-6 band)", B);

    /* y against the oracle's sparse FFN over the same list (the oracle's own list when the GPU's
     * failed its checks, so that no out-of-range id is read) */
    orc_sparse_ffn(ORC_F16, ORC_RELU, D, F, w_up, NULL, NULL, NULL, w_dT, NULL, b_up, NULL, b_down, ORC_F16, x, B,
                   set_ok ? idx : idx_ref, set_ok ? n : n_ref, y_ref);
    double ymax = 0.0, yerr = 0.0;
    for (int i = 0; i < B * D; ++i) {
      ymax = fmax(ymax, fabs(y_ref[i]));
      yerr = fmax(yerr, fabs((double)y[i] - y_ref[i]));
    }
    check(ymax > 0.0 && yerr <= 2e-3 * ymax, "y within 2e-3 (relative to max |y|) of the oracle", B);
    printf("     B=%d: %d of %d neurons active, max |dlogit| %.2e, max |dy| / max |y| %.2e\n", B, n, F, lerr,
           ymax > 0.0 ? yerr / ymax : 0.0);
  }
  hipFree(ws);
  hipFree(didx);
  hipFree(dcount);
  hipFree(dlogits);
  hipFree(dy);
  hipFree(dx);
  hipFree((void*)P.A);
  hipFree((void*)P.Q);
  hipFree((void*)P.c);
  hipFree((void*)W.w_up);
  hipFree((void*)W.w_dT);
  hipFree((void*)W.b_up);
  hipFree((void*)W.b_down);
  printf("%d failed\n", failed);
  return failed;
}

/*
 * A plain C11 caller of libpsffn's ABI (include/psffn.h), built by tests/test_c_consumer_host.py
 * with gcc and linked against the in-tree library.  Host side only: every call that takes device
 * pointers carries at least one invalid argument, so the library's validation returns before any
 * HIP call and the fake addresses below are never dereferenced or handed to a kernel.
 * Prints one line per check and exits with the number of failed checks.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "psffn.h"

static int failed = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failed;
}

/* suitably aligned fake device addresses: validation never dereferences them */
static const void* fake(unsigned k) { return (const void*)(uintptr_t)(0x7F0000000000ull + ((uintptr_t)k << 28)); }

int main(void) {
  /* a predictor and an FFN shaped like the OPT-30B layer (d 7168, F 28672, r 1024, fp16 ReLU) */
  psffn_predictor P;
  memset(&P, 0, sizeof P);
  P.d = 7168;
  P.F = 28672;
  P.r = 1024;
  P.dt = PSFFN_F16;
  P.A = fake(1);
  P.Q = fake(2);
  P.c = (const float*)fake(3);

  psffn_ffn W;
  memset(&W, 0, sizeof W);
  W.d = 7168;
  W.F = 28672;
  W.dt = PSFFN_F16;
  W.act = PSFFN_RELU;
  W.w_up = fake(4);
  W.w_dT = fake(5);
  W.b_up = (const float*)fake(6);

  /* status strings: one per status, all distinct */
  const psffn_status all[] = {PSFFN_OK, PSFFN_E_INVALID_ARG, PSFFN_E_UNSUPPORTED, PSFFN_E_WORKSPACE, PSFFN_E_HIP};
  int distinct = 1;
  for (int i = 0; i < 5; ++i) {
    if (!psffn_status_str(all[i]) || !psffn_status_str(all[i])[0]) distinct = 0;
    for (int j = 0; j < i; ++j)
      if (psffn_status_str(all[i]) && psffn_status_str(all[j]) && strcmp(psffn_status_str(all[i]), psffn_status_str(all[j])) == 0)
        distinct = 0;
  }
  check(distinct, "psffn_status_str: a distinct non-empty string per status");

  /* workspace sizes */
  const size_t n_pred = psffn_workspace_bytes(&P, NULL, 1);
  const size_t n_layer = psffn_workspace_bytes(&P, &W, 1);
  const size_t n_layer8 = psffn_workspace_bytes(&P, &W, 8);
  check(n_pred > 0 && n_pred <= n_layer && n_layer < n_layer8, "psffn_workspace_bytes: predictor <= layer < layer at 8 tokens");
  check(psffn_workspace_bytes(NULL, NULL, 1) == 0, "psffn_workspace_bytes: no descriptor gives 0");
  check(psffn_workspace_bytes(&P, &W, 0) == 0 && psffn_workspace_bytes(&P, &W, PSFFN_MAX_BATCH + 1) == 0,
        "psffn_workspace_bytes: batch outside 1..PSFFN_MAX_BATCH gives 0");

  /* argument checks before anything is enqueued */
  int32_t* idx = (int32_t*)fake(7);
  int32_t* count = (int32_t*)fake(8);
  float* y = (float*)fake(9);
  void* ws = (void*)fake(10);
  check(psffn_predict(NULL, fake(11), 1, 0.0f, idx, count, NULL, ws, n_pred, NULL) == PSFFN_E_INVALID_ARG,
        "psffn_predict: no predictor -> PSFFN_E_INVALID_ARG");
  check(psffn_predict(&P, fake(11), 0, 0.0f, idx, count, NULL, ws, n_pred, NULL) == PSFFN_E_INVALID_ARG,
        "psffn_predict: batch 0 -> PSFFN_E_INVALID_ARG");
  check(psffn_predict(&P, fake(11), 1, nanf(""), idx, count, NULL, ws, n_pred, NULL) == PSFFN_E_INVALID_ARG,
        "psffn_predict: NaN threshold -> PSFFN_E_INVALID_ARG");
  check(psffn_predict(&P, fake(11), 1, 0.0f, idx, count, NULL, ws, n_pred - 1, NULL) == PSFFN_E_WORKSPACE,
        "psffn_predict: workspace one byte short -> PSFFN_E_WORKSPACE");
  check(psffn_layer(&P, &W, fake(11), 1, 0.0f, idx, count, NULL, y, 0, NULL, n_layer, NULL) == PSFFN_E_WORKSPACE,
        "psffn_layer: no workspace -> PSFFN_E_WORKSPACE");

  psffn_ffn W4 = W;
  W4.dt = PSFFN_I4G128;
  W4.d = 7168 + 64; /* 4-bit rows need d % 128 == 0 */
  check(psffn_sparse_ffn(&W4, fake(11), 1, idx, count, y, 0, ws, n_layer, NULL) == PSFFN_E_UNSUPPORTED,
        "psffn_sparse_ffn: 4-bit rows with d % 128 != 0 -> PSFFN_E_UNSUPPORTED");
  psffn_ffn Wg = W;
  Wg.act = PSFFN_SWIGLU; /* no gate rows */
  check(psffn_sparse_ffn(&Wg, fake(11), 1, idx, count, y, 0, ws, n_layer, NULL) == PSFFN_E_INVALID_ARG,
        "psffn_sparse_ffn: SwiGLU without gate rows -> PSFFN_E_INVALID_ARG");
  check(psffn_workspace_init(NULL, 1024, NULL) == PSFFN_E_WORKSPACE, "psffn_workspace_init: no workspace -> PSFFN_E_WORKSPACE");

  printf("%d failed\n", failed);
  return failed;
}

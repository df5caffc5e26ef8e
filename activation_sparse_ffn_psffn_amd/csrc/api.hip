// extern "C" boundary of libpsffn: argument validation (host only, before anything is enqueued),
// workspace layout, and dispatch to the launchers.  See include/psffn.h for the contract.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "common.h"

using namespace psffn;

// Scratch of psffn_layer_noalloc: the workspace of that call lives here, one copy per GPU (each
// device holds its own instance of this array at its own address, for as long as the process runs).
// Host code never uses the array's name as an address: it takes the device address of the current
// GPU's copy from hipGetSymbolAddress once per device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[PSFFN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch; on the first call for a device, the address is
// looked up and the scratch cleared with the fill kernel on the caller's stream (no memset node).
psffn_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PSFFN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PSFFN_E_HIP;
    if (launch_fill_zero(p, PSFFN_NOALLOC_SCRATCH_BYTES, stream) != hipSuccess) return PSFFN_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PSFFN_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// An enum field as the int a C caller stored in it (any value: reading a C++ enum object that holds a
// value outside the enumeration's range would be undefined behaviour, so it is copied out as bytes).
template <class E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

St st_of(psffn_dtype dt) { return dt == PSFFN_F32 ? St::F32 : (dt == PSFFN_F16 ? St::F16 : St::I4); }

size_t elem_row_bytes(psffn_dtype dt, int n) {
  return dt == PSFFN_F32 ? (size_t)n * 4 : (dt == PSFFN_F16 ? (size_t)n * 2 : (size_t)n / 2);
}

bool batch_ok(int B) { return B >= 1 && B <= PSFFN_MAX_BATCH; }

psffn_status check_pred(const psffn_predictor* P) {
  if (!P) return PSFFN_E_INVALID_ARG;
  if (P->d <= 0 || P->F <= 0 || P->r <= 0) return PSFFN_E_INVALID_ARG;
  if (P->d > kMaxD || P->r > kMaxD) return PSFFN_E_UNSUPPORTED;
  const int dt = enum_value(P->dt);
  if (dt != PSFFN_F32 && dt != PSFFN_F16) return PSFFN_E_UNSUPPORTED;
  if (P->d % 8 != 0 || P->r % 8 != 0) return PSFFN_E_UNSUPPORTED;
  if (!P->A || !P->Q || !P->c) return PSFFN_E_INVALID_ARG;
  if (!aligned(P->A, 16) || !aligned(P->Q, 16) || !aligned(P->c, 4)) return PSFFN_E_INVALID_ARG;
  return PSFFN_OK;
}

psffn_status check_ffn(const psffn_ffn* W) {
  if (!W) return PSFFN_E_INVALID_ARG;
  if (W->d <= 0 || W->F <= 0) return PSFFN_E_INVALID_ARG;
  if (W->d > kMaxD) return PSFFN_E_UNSUPPORTED;
  const int dt = enum_value(W->dt), act = enum_value(W->act);
  if (dt != PSFFN_F32 && dt != PSFFN_F16 && dt != PSFFN_I4G128) return PSFFN_E_UNSUPPORTED;
  if (act != PSFFN_RELU && act != PSFFN_SWIGLU) return PSFFN_E_UNSUPPORTED;
  if (W->dt == PSFFN_I4G128 ? (W->d % 128 != 0) : (W->d % 8 != 0)) return PSFFN_E_UNSUPPORTED;
  if (!W->w_up || !W->w_dT) return PSFFN_E_INVALID_ARG;
  if (!aligned(W->w_up, 16) || !aligned(W->w_dT, 16)) return PSFFN_E_INVALID_ARG;
  if (W->act == PSFFN_SWIGLU && (!W->w_gate || !aligned(W->w_gate, 16))) return PSFFN_E_INVALID_ARG;
  if (W->dt == PSFFN_I4G128) {
    if (!W->s_up || !W->s_dT || !aligned(W->s_up, 2) || !aligned(W->s_dT, 2)) return PSFFN_E_INVALID_ARG;
    if (W->act == PSFFN_SWIGLU && (!W->s_gate || !aligned(W->s_gate, 2))) return PSFFN_E_INVALID_ARG;
  }
  if ((W->b_up && !aligned(W->b_up, 4)) || (W->b_gate && !aligned(W->b_gate, 4)) ||
      (W->b_down && !aligned(W->b_down, 4)))
    return PSFFN_E_INVALID_ARG;
  return PSFFN_OK;
}

// per-call scratch sizes (after the reserved state head)
size_t predict_scratch(int B, int r, int F) { return round256((size_t)B * r * 4) + round256((size_t)F + 16); }
size_t compact_scratch(int F) { return round256((size_t)F + 16); }
size_t ffn_scratch(int B, int d, int F) {
  const size_t splits = kUDSplitCap > kSplitCap ? kUDSplitCap : kSplitCap;
  return round256((size_t)F * B * 4) + round256(splits * B * (size_t)d * 4);
}

// scratch of a call, whichever pipeline its batch size takes
size_t pred_need(const psffn_predictor& P, int B) {
  size_t v = predict_scratch(B, P.r, P.F);
  if (batch_supported_pred(P, B)) {
    const size_t b = batch_scratch_bytes(B, P.d, P.r, P.F, PSFFN_F16, PSFFN_RELU, true, false);
    v = b > v ? b : v;
  }
  return v;
}
size_t ffn_need(const psffn_ffn& W, int B) {
  size_t v = ffn_scratch(B, W.d, W.F);
  if (batch_supported_ffn(W, B)) {
    const size_t b = batch_scratch_bytes(B, W.d, 0, W.F, W.dt, W.act, false, true);
    v = b > v ? b : v;
  }
  return v;
}

// Pipeline choice for 2..kFusedMaxBatch tokens, per stage (measured on MI355X at B = 2..4: the
// MFMA batch pipeline's cost hardly grows with the batch, the small-batch kernels' per-token work
// does).  Each stage's choice depends on its own descriptor and B only, so that psffn_layer gives
// exactly the outputs of psffn_predict followed by psffn_sparse_ffn.
//  * predictor: the batch pipeline from 3 tokens, and at 2 tokens above 1024 ranks (the
//    small-batch logits kernel then holds three slices of h per token and lane);
//  * FFN: the batch pipeline for 4-bit weights from 2 tokens and for fp16 ReLU weights from 3;
//    fp16 SwiGLU layers (about half the neurons active, so the FFN dominates) stream their rows
//    faster through the small-batch kernel.
// Above kFusedMaxBatch tokens only the batch pipeline exists.
bool pred_on_batch(const psffn_predictor& P, int B) {
  if (B > kFusedMaxBatch) return true;
  if (!batch_supported_pred(P, B)) return false;
  return B >= 3 || P.r > 1024;
}

bool ffn_on_batch(const psffn_ffn& W, int B) {
  if (B > kFusedMaxBatch) return true;
  if (!batch_supported_ffn(W, B)) return false;
  if (W.dt == PSFFN_I4G128) return true;
  return W.act == PSFFN_RELU && B >= 3;
}

psffn_status check_ws(const void* ws, size_t ws_bytes, int F, size_t need) {
  if (!ws || !aligned(ws, 256) || ws_bytes < state_layout(F).scratch + need) return PSFFN_E_WORKSPACE;
  return PSFFN_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

psffn_status hip_status(hipError_t e) { return e == hipSuccess ? PSFFN_OK : PSFFN_E_HIP; }

// every argument of a layer call except the workspace
psffn_status layer_args_ok(const psffn_predictor* P, const psffn_ffn* W, int n_hot, const void* x, int B,
                           float logit_thr, const int32_t* idx, const int32_t* count, const float* logits,
                           const float* y) {
  psffn_status st = check_pred(P);
  if (st == PSFFN_OK) st = check_ffn(W);
  if (st != PSFFN_OK) return st;
  if (n_hot < 0 || n_hot > P->F) return PSFFN_E_INVALID_ARG;
  if (P->F != W->F || P->d != W->d) return PSFFN_E_INVALID_ARG;
  if ((P->dt == PSFFN_F32) != (W->dt == PSFFN_F32)) return PSFFN_E_UNSUPPORTED;
  if (!batch_ok(B) || !x || !aligned(x, 16) || !idx || !aligned(idx, 4) || !count || !aligned(count, 4) || !y ||
      !aligned(y, 4) || (logits && !aligned(logits, 4)) || logit_thr != logit_thr)
    return PSFFN_E_INVALID_ARG;
  return PSFFN_OK;
}

}  // namespace

extern "C" {

const char* psffn_status_str(psffn_status s) {
  switch (enum_value(s)) {
    case PSFFN_OK: return "ok";
    case PSFFN_E_INVALID_ARG: return "invalid argument";
    case PSFFN_E_UNSUPPORTED: return "unsupported dtype/activation/shape combination";
    case PSFFN_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case PSFFN_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t psffn_workspace_bytes(const psffn_predictor* P, const psffn_ffn* W, int B) {
  if (!batch_ok(B) || (!P && !W)) return 0;
  if (P && check_pred(P) != PSFFN_OK) return 0;
  if (W && check_ffn(W) != PSFFN_OK) return 0;
  if (P && W && P->F != W->F) return 0;
  const int F = P ? P->F : W->F;
  size_t need = compact_scratch(F);
  if (P) {
    size_t v = pred_need(*P, B);
    need = v > need ? v : need;
  }
  if (W) {
    size_t v = ffn_need(*W, B);
    need = v > need ? v : need;
  }
  return state_layout(F).scratch + need;
}

psffn_status psffn_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned(ws, 256) || ws_bytes == 0 || ws_bytes % 16 != 0) return PSFFN_E_WORKSPACE;
  return hip_status(launch_fill_zero(ws, ws_bytes, stream));
}

psffn_status psffn_predict(const psffn_predictor* P, const void* x, int B, float logit_thr, int32_t* idx,
                           int32_t* count, float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  return psffn_predict_hot(P, 0, x, B, logit_thr, idx, count, logits, ws, ws_bytes, stream);
}

psffn_status psffn_predict_hot(const psffn_predictor* P, int n_hot, const void* x, int B, float logit_thr,
                               int32_t* idx, int32_t* count, float* logits, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  psffn_status st = check_pred(P);
  if (st != PSFFN_OK) return st;
  if (n_hot < 0 || n_hot > P->F) return PSFFN_E_INVALID_ARG;
  if (!batch_ok(B) || !x || !aligned(x, 16) || !idx || !aligned(idx, 4) || !count || !aligned(count, 4) ||
      (logits && !aligned(logits, 4)) || logit_thr != logit_thr)
    return PSFFN_E_INVALID_ARG;
  st = check_ws(ws, ws_bytes, P->F, pred_need(*P, B));
  if (st != PSFFN_OK) return st;
  const St pt = st_of(P->dt);
  hipError_t e = hipErrorNotSupported;
  if (pred_on_batch(*P, B))
    e = launch_predict_batch(*P, x, B, logit_thr, idx, count, logits, ws, stream, n_hot);
  if (e == hipErrorNotSupported && B <= kFusedMaxBatch)
    e = launch_predict_fused(pt, *P, x, B, logit_thr, idx, count, logits, ws, stream, n_hot);
  if (e == hipErrorNotSupported) {
    char* base = static_cast<char*>(ws) + state_layout(P->F).scratch;
    float* h = reinterpret_cast<float*>(base);
    uint8_t* flags = reinterpret_cast<uint8_t*>(base + round256((size_t)B * P->r * 4));
    e = launch_pred_h(pt, P->A, x, B, P->d, P->r, h, stream);
    if (e == hipSuccess) e = launch_pred_logits(pt, P->Q, P->c, h, B, P->r, P->F, logit_thr, logits, flags, stream);
    if (e == hipSuccess) e = launch_scatter(flags, P->F, idx, count, stream, n_hot);
  }
  return hip_status(e);
}

psffn_status psffn_compact(const float* logits, int B, int F, float logit_thr, int32_t* idx, int32_t* count,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!batch_ok(B) || F <= 0 || !logits || !aligned(logits, 4) || !idx || !aligned(idx, 4) || !count ||
      !aligned(count, 4) || logit_thr != logit_thr)
    return PSFFN_E_INVALID_ARG;
  psffn_status st = check_ws(ws, ws_bytes, F, compact_scratch(F));
  if (st != PSFFN_OK) return st;
  uint8_t* flags = static_cast<uint8_t*>(ws) + state_layout(F).scratch;
  hipError_t e = launch_flags_from_logits(logits, B, F, logit_thr, flags, stream);
  if (e == hipSuccess) e = launch_scatter(flags, F, idx, count, stream);
  return hip_status(e);
}

psffn_status psffn_sparse_ffn(const psffn_ffn* W, const void* x, int B, const int32_t* idx, const int32_t* count,
                              float* y, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
  psffn_status st = check_ffn(W);
  if (st != PSFFN_OK) return st;
  if (!batch_ok(B) || !x || !aligned(x, 16) || !idx || !aligned(idx, 4) || !count || !aligned(count, 4) || !y ||
      !aligned(y, 4))
    return PSFFN_E_INVALID_ARG;
  st = check_ws(ws, ws_bytes, W->F, ffn_need(*W, B));
  if (st != PSFFN_OK) return st;
  const St wt = st_of(W->dt);
  hipError_t e = hipErrorNotSupported;
  if (ffn_on_batch(*W, B)) e = launch_ffn_batch(*W, x, B, idx, count, y, accumulate, ws, stream);
  else if (stream_ffn_fits(*W, B) || stream_ffn_i4_fits(*W, B))
    e = launch_ffn_stream(*W, x, idx, count, y, accumulate, ws, stream);
  if (e == hipErrorNotSupported && B <= kFusedMaxBatch)
    e = launch_ffn_fused(wt, *W, x, B, idx, count, y, accumulate, ws, stream);
  if (e == hipErrorNotSupported) {
    char* base = static_cast<char*>(ws) + state_layout(W->F).scratch;
    float* a = reinterpret_cast<float*>(base);
    float* part = reinterpret_cast<float*>(base + round256((size_t)W->F * B * 4));
    e = launch_up(wt, W->act, *W, x, B, idx, count, a, stream);
    if (e == hipSuccess) e = launch_down(wt, *W, a, B, idx, count, part, stream);
    if (e == hipSuccess) e = launch_reduce(part, count, W->F, B, W->d, W->b_down, y, accumulate, stream);
  }
  return hip_status(e);
}

psffn_status psffn_layer(const psffn_predictor* P, const psffn_ffn* W, const void* x, int B, float logit_thr,
                         int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  return psffn_layer_hot(P, W, 0, x, B, logit_thr, idx, count, logits, y, accumulate, ws, ws_bytes, stream);
}

psffn_status psffn_layer_hot(const psffn_predictor* P, const psffn_ffn* W, int n_hot, const void* x, int B,
                             float logit_thr, int32_t* idx, int32_t* count, float* logits, float* y, int accumulate,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  psffn_status st = layer_args_ok(P, W, n_hot, x, B, logit_thr, idx, count, logits, y);
  if (st != PSFFN_OK) return st;
  size_t need = pred_need(*P, B);
  const size_t f = ffn_need(*W, B);
  need = f > need ? f : need;
  st = check_ws(ws, ws_bytes, W->F, need);
  if (st != PSFFN_OK) return st;
  hipError_t e = hipErrorNotSupported;
  const bool pb = pred_on_batch(*P, B), fb = ffn_on_batch(*W, B);
  if (!pb && !fb && stream_layer_fits(*P, *W, B, false) && stream_scratch(P->r, P->F, P->d) <= need) {
    // one token, fp16 or 4-bit ReLU: up rows inside the logits kernel, the split sum inside the down kernel
    e = launch_layer_stream(*P, *W, x, logit_thr, idx, count, logits, y, accumulate, ws, stream, n_hot, LnArgs{});
  } else if (pb && fb) {
    e = launch_layer_batch(*P, *W, x, B, logit_thr, idx, count, logits, y, accumulate, ws, stream, n_hot);
  } else if (!pb && !fb) {
    e = launch_layer_fused(*P, *W, x, B, logit_thr, idx, count, logits, y, accumulate, ws, stream, n_hot);
  } else if (pb && ffn_fused_scan_fits(*W, B)) {
    // batch predictor up to its mask words, then the small-batch FFN orders the list from them (the
    // list the batch predictor's own list kernel would write, so the outputs equal the two calls)
    e = launch_predict_batch_masks(*P, x, B, logit_thr, logits, ws, stream);
    if (e == hipSuccess)
      e = launch_ffn_fused_scan(st_of(W->dt), *W, x, B, idx, count, y, accumulate, ws, stream, n_hot);
  }
  if (e != hipErrorNotSupported) return hip_status(e);
  // shapes outside the one-call paths: the two calls, same results
  st = psffn_predict_hot(P, n_hot, x, B, logit_thr, idx, count, logits, ws, ws_bytes, stream);
  if (st != PSFFN_OK) return st;
  return psffn_sparse_ffn(W, x, B, idx, count, y, accumulate, ws, ws_bytes, stream);
}

psffn_status psffn_layer_noalloc(const psffn_predictor* P, const psffn_ffn* W, const void* x, int B,
                                 float logit_thr, int32_t* idx, int32_t* count, float* logits, float* y,
                                 int accumulate, hipStream_t stream) {
  // every argument is checked before anything (the first call's clearing of the scratch included)
  // is enqueued; the scratch this call needs (psffn_layer's workspace) must fit the static array
  const psffn_status chk = layer_args_ok(P, W, 0, x, B, logit_thr, idx, count, logits, y);
  if (chk != PSFFN_OK) return chk;
  const size_t need = psffn_workspace_bytes(P, W, B);
  if (need == 0 || need > (size_t)PSFFN_NOALLOC_SCRATCH_BYTES) return PSFFN_E_WORKSPACE;
  void* ws = nullptr;
  const psffn_status st = noalloc_scratch(stream, &ws);
  if (st != PSFFN_OK) return st;
  return psffn_layer(P, W, x, B, logit_thr, idx, count, logits, y, accumulate, ws,
                     (size_t)PSFFN_NOALLOC_SCRATCH_BYTES, stream);
}

psffn_status psffn_layer_ln(const psffn_predictor* P, const psffn_ffn* W, float* x, float eps, void* h, int B,
                            float logit_thr, int32_t* idx, int32_t* count, float* logits, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  psffn_status st = check_pred(P);
  if (st == PSFFN_OK) st = check_ffn(W);
  if (st != PSFFN_OK) return st;
  if (P->F != W->F || P->d != W->d) return PSFFN_E_INVALID_ARG;
  if (P->dt != PSFFN_F16) return PSFFN_E_UNSUPPORTED;  // the LayerNorm output (the FFN input) is fp16
  const int d = P->d;
  if (!batch_ok(B) || !x || !aligned(x, 16) || !h || !aligned(h, 16) || !idx || !aligned(idx, 4) || !count ||
      !aligned(count, 4) || (logits && !aligned(logits, 4)) || logit_thr != logit_thr || !(eps >= 0.f) ||
      overlaps(x, (size_t)B * d * 4, h, (size_t)B * d * 2))
    return PSFFN_E_INVALID_ARG;
  size_t need = pred_need(*P, B);
  const size_t f = ffn_need(*W, B);
  need = f > need ? f : need;
  st = check_ws(ws, ws_bytes, W->F, need);
  if (st != PSFFN_OK) return st;
  hipError_t e = hipErrorNotSupported;
  LnArgs ln;
  ln.xres = x;
  ln.eps = eps;
  ln.hout = static_cast<_Float16*>(h);
  const bool small = B <= kFusedMaxBatch && !pred_on_batch(*P, B) && !ffn_on_batch(*W, B);
  if (small && stream_layer_fits(*P, *W, B, true) && stream_scratch(P->r, P->F, P->d) <= need) {
    e = launch_layer_stream(*P, *W, h, logit_thr, idx, count, logits, x, 1, ws, stream, 0, ln);
  } else if (small && !stream_ffn_i4_fits(*W, B)) {
    e = launch_layer_fused(*P, *W, h, B, logit_thr, idx, count, logits, x, 1, ws, stream, 0, ln);
  }
  if (e != hipErrorNotSupported) return hip_status(e);
  // the other pipelines: the LayerNorm kernel, then the layer call (the same results)
  e = launch_layernorm_f16(x, B, d, eps, h, stream);
  if (e != hipSuccess) return hip_status(e);
  return psffn_layer(P, W, h, B, logit_thr, idx, count, logits, x, 1, ws, ws_bytes, stream);
}

psffn_status psffn_profile_counts(const psffn_ffn* W, const void* X, int T, int32_t* counts, hipStream_t stream) {
  psffn_status st = check_ffn(W);
  if (st != PSFFN_OK) return st;
  if (T < 1 || !X || !aligned(X, 16) || !counts || !aligned(counts, 4)) return PSFFN_E_INVALID_ARG;
  return hip_status(launch_profile_counts(st_of(W->dt), *W, X, T, counts, stream));
}

psffn_status psffn_permute_hot_first(const int32_t* counts, int F, int32_t* perm, const psffn_ffn* src,
                                     const psffn_ffn* dst, const psffn_predictor* psrc, const psffn_predictor* pdst,
                                     hipStream_t stream) {
  if (F <= 0 || !counts || !aligned(counts, 4) || !perm || !aligned(perm, 4)) return PSFFN_E_INVALID_ARG;
  if ((src == nullptr) != (dst == nullptr) || (psrc == nullptr) != (pdst == nullptr)) return PSFFN_E_INVALID_ARG;
  struct Job {
    const void* s;
    void* t;
    size_t rb;
  } jobs[12];
  int nj = 0;
  auto add = [&](const void* s, const void* t, size_t rb) -> bool {
    if (!s && !t) return true;
    if (!s || !t) return false;
    if (overlaps(s, rb * F, t, rb * F)) return false;
    jobs[nj++] = Job{s, const_cast<void*>(t), rb};
    return true;
  };
  if (src) {
    psffn_status st = check_ffn(src);
    if (st == PSFFN_OK) st = check_ffn(dst);
    if (st != PSFFN_OK) return st;
    if (src->F != F || dst->F != F || src->d != dst->d || src->dt != dst->dt || src->act != dst->act)
      return PSFFN_E_INVALID_ARG;
    const size_t rb = elem_row_bytes(src->dt, src->d);
    const size_t sb = src->dt == PSFFN_I4G128 ? (size_t)(src->d / 128) * 2 : 0;
    bool ok = add(src->w_up, dst->w_up, rb) && add(src->w_dT, dst->w_dT, rb) &&
              (src->act != PSFFN_SWIGLU || add(src->w_gate, dst->w_gate, rb)) &&
              add(src->b_up, dst->b_up, 4) && add(src->b_gate, dst->b_gate, 4);
    if (ok && sb) {
      ok = add(src->s_up, dst->s_up, sb) && add(src->s_dT, dst->s_dT, sb) &&
           (src->act != PSFFN_SWIGLU || add(src->s_gate, dst->s_gate, sb));
    }
    if (!ok) return PSFFN_E_INVALID_ARG;
  }
  if (psrc) {
    psffn_status st = check_pred(psrc);
    if (st == PSFFN_OK) st = check_pred(pdst);
    if (st != PSFFN_OK) return st;
    if (psrc->F != F || pdst->F != F || psrc->r != pdst->r || psrc->d != pdst->d || psrc->dt != pdst->dt)
      return PSFFN_E_INVALID_ARG;
    if (!add(psrc->Q, pdst->Q, elem_row_bytes(psrc->dt, psrc->r)) || !add(psrc->c, pdst->c, 4))
      return PSFFN_E_INVALID_ARG;
  }
  hipError_t e = launch_hot_first_perm(counts, F, perm, stream);
  for (int j = 0; j < nj && e == hipSuccess; ++j) e = launch_gather_rows(jobs[j].s, jobs[j].t, perm, F, jobs[j].rb, stream);
  return hip_status(e);
}

psffn_status psffn_layernorm_f16(const float* x, int B, int d, float eps, void* out_f16, hipStream_t stream) {
  if (B < 1 || d < 1 || !x || !aligned(x, 4) || !out_f16 || !aligned(out_f16, 2) || !(eps >= 0.f))
    return PSFFN_E_INVALID_ARG;
  return hip_status(launch_layernorm_f16(x, B, d, eps, out_f16, stream));
}

}  // extern "C"

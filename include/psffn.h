/*
 * psffn.h -- C ABI of libpsffn: predictor-gated, neuron-level sparse FFN for decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU",
 * Elamur Research summary):
 *   - Summary, 1st paragraph: MLP activations follow a power law -- a few hot neurons fire
 *     for most inputs, a long tail of cold neurons only for specific inputs.
 *   - Summary, 2nd paragraph: a lightweight predictor per layer guesses which neurons will
 *     fire; neuron-level kernels compute those and skip the rest; neurons are profiled
 *     offline by how often they fire.
 *   - Interesting ideas, I4: the kernels operate directly on weight rows and columns, with no
 *     sparse-format conversion.
 *   - Interesting ideas, I1: the most used neurons are placed first / in the fastest memory.
 *   - Key points (sparsity): ReLU MLPs (OPT) are ~97% sparse, SwiGLU ones (LLaMA2) ~43%.
 *   - Summary, 1st paragraph and Key points (speed): models also run 4-bit quantised.
 *
 * Readings where the pages are silent (they give no predictor form, threshold, layout or
 * 4-bit format):
 *   - predictor: linear low rank, h = A x (A: r x d), logit l = Q h + c (Q: F x r); neuron i
 *     is predicted to fire when sigmoid(l_i) > tau, i.e. l_i > logit(tau); tau = 1/2 gives 0;
 *   - a batch of B tokens shares ONE neuron list: the union of the per-token predicted sets;
 *   - ReLU FFN:   a_i = max(W_up[i].x + b_up[i], 0)
 *     SwiGLU FFN: a_i = silu(W_gate[i].x + b_gate[i]) * (W_up[i].x + b_up[i])
 *     output:     y = b_down + sum over listed i of a_i * W_dT[i]   (W_dT = W_down transposed)
 *   - 4-bit weights: per row, element 2j in the low nibble of byte j, element 2j+1 in the high
 *     nibble, each a two's-complement integer in [-8, 7] multiplied by the fp16 scale of its
 *     group of 128 consecutive elements.
 *
 * Conventions for every call:
 *   - All matrices are row-major and NEURON-MAJOR: row i of w_up, w_gate, w_dT and Q belongs
 *     to neuron i, so a neuron's weights are contiguous rows (Interesting ideas, I4).
 *   - Every pointer named in a descriptor or argument is a DEVICE pointer unless stated, owned
 *     by the caller, 16-byte aligned (the workspace: 256-byte aligned).  The library never
 *     allocates or frees memory, never synchronises the stream, and enqueues all work on the
 *     given stream; calls with distinct workspaces are independent and thread-safe.
 *   - Host-side validation runs before anything is enqueued.  On any error nothing is
 *     enqueued and no output is written.  No C++ exception crosses the ABI.
 *   - Activations x: fp32 [B][d] when the weights are PSFFN_F32, else fp16 [B][d].
 *     h, logits, activations and y are fp32.  Biases are fp32 and may be NULL (= zero).
 *   - Batch: 1 <= B <= PSFFN_MAX_BATCH.
 */
#ifndef PSFFN_H_
#define PSFFN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSFFN_MAX_BATCH 32

typedef enum {
  PSFFN_OK = 0,
  PSFFN_E_INVALID_ARG = 1,  /* null/misaligned pointer, non-positive size, B out of range */
  PSFFN_E_UNSUPPORTED = 2,  /* dtype / activation / shape combination not provided */
  PSFFN_E_WORKSPACE = 3,    /* workspace missing, misaligned or smaller than required */
  PSFFN_E_HIP = 4           /* a HIP launch failed; the HIP error is left for hipGetLastError */
} psffn_status;

typedef enum {
  PSFFN_F32 = 0,    /* fp32 */
  PSFFN_F16 = 1,    /* IEEE binary16 */
  PSFFN_I4G128 = 2  /* 4-bit weights + fp16 scale per 128 elements (FFN weights only) */
} psffn_dtype;

typedef enum { PSFFN_RELU = 0, PSFFN_SWIGLU = 1 } psffn_act;

/* Low-rank activation predictor of one layer.  dt is PSFFN_F32 or PSFFN_F16 (A and Q share it;
 * a 4-bit layer keeps an fp16 predictor).  Requirements: d % 8 == 0 and r % 8 == 0. */
typedef struct {
  int d, F, r;
  psffn_dtype dt;
  const void* A;   /* [r][d] */
  const void* Q;   /* [F][r] */
  const float* c;  /* [F], required */
} psffn_predictor;

/* FFN weights of one layer, neuron-major.
 *   dt = PSFFN_F32 / PSFFN_F16: w_* are [F][d] of that type, s_* unused (NULL).
 *   dt = PSFFN_I4G128:          w_* are uint8 [F][d/2] (packed nibbles), s_* fp16 [F][d/128].
 *   act = PSFFN_RELU uses w_up (+ b_up); act = PSFFN_SWIGLU also needs w_gate (+ b_gate).
 * Requirements: d % 8 == 0 (dense) or d % 128 == 0 (4-bit). */
typedef struct {
  int d, F;
  psffn_dtype dt;
  psffn_act act;
  const void* w_up;
  const void* w_gate;
  const void* w_dT;     /* W_down transposed: row i = output weights of neuron i */
  const void* s_up;
  const void* s_gate;
  const void* s_dT;
  const float* b_up;    /* [F] or NULL */
  const float* b_gate;  /* [F] or NULL (SwiGLU) */
  const float* b_down;  /* [d] or NULL */
} psffn_ffn;

/* Bytes of workspace needed by any call below for these shapes (either descriptor may be
 * NULL).  Returns 0 when the arguments are invalid. */
size_t psffn_workspace_bytes(const psffn_predictor* P, const psffn_ffn* W, int B);

/* Zero-fill a workspace with a device kernel (no memset node, so it can be captured in a
 * graph).  A workspace must be initialised once before its first use; every call leaves it
 * initialised again on return, so it can be reused by any later call on the same stream.
 * Calls that share a workspace must be ordered on one stream. */
psffn_status psffn_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Predict and compact (Summary, 2nd paragraph: per-layer predictors guess which neurons fire).
 *   x      [B][d] activations (fp32 if P->dt == PSFFN_F32, else fp16)
 *   logit_thr  threshold on the logit (tau = 1/2 -> 0.0f); a neuron is active for the batch when
 *          Q_i.(A x_b) + c_i > logit_thr for at least one b (strict)
 *   idx    out, int32 [F]: the active neurons in ascending order; entries past *count are
 *          left unspecified
 *   count  out, one int32 in device memory: number of active neurons (stays on the device)
 *   logits out, optional fp32 [B][F] (NULL to skip)
 *   h is kept in fp32 between the two predictor stages. */
psffn_status psffn_predict(const psffn_predictor* P, const void* x, int B, float logit_thr, int32_t* idx,
                           int32_t* count, float* logits, void* ws, size_t ws_bytes, hipStream_t stream);

/* Threshold + compaction alone (Summary, 2nd paragraph: the kernels compute the neurons the
 * predictor keeps and skip the rest -- this call forms the kept list), on logits produced
 * elsewhere: logits fp32 [B][F] -> ascending idx [F] and count (same rules as psffn_predict:
 * neuron i is kept when logits[b][i] > logit_thr for at least one b). */
psffn_status psffn_compact(const float* logits, int B, int F, float logit_thr, int32_t* idx, int32_t* count,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Sparse FFN over a neuron list (Summary, 2nd paragraph: compute the predicted neurons and skip
 * the rest; Interesting ideas, I4: whole weight rows, no sparse format).
 *   idx/count  any list of distinct neuron indices in [0, F) (device memory; count in [0, F]),
 *              e.g. the output of psffn_predict; every token of the batch uses the same list.
 *   y          out, fp32 [B][d]: y_b = b_down + sum_k a_{idx[k]}(x_b) * W_dT[idx[k]]
 *              (accumulate != 0: y_b += that instead, e.g. a residual stream).
 * The summation order is a fixed function of (idx, count, shapes): repeated calls give
 * bit-identical y.  With count == 0, y = b_down (or y unchanged plus b_down). */
psffn_status psffn_sparse_ffn(const psffn_ffn* W, const void* x, int B, const int32_t* idx, const int32_t* count,
                              float* y, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* One decode step of one layer: psffn_predict followed by psffn_sparse_ffn on its list, with
 * the same outputs (idx ascending, count, optional logits, y, bit for bit) and the same
 * requirements, in the fewest launches: at one token with fp16 or 4-bit ReLU weights the up rows are
 * computed inside the predictor's logits kernel and the list is written by the down projection;
 * elsewhere the list is ordered inside the FFN's first kernel instead of by the predictor.
 * P and W must describe the same layer (same F and d); P->dt is fp32 exactly when W->dt is fp32. */
psffn_status psffn_layer(const psffn_predictor* P, const psffn_ffn* W, const void* x, int B, float logit_thr,
                         int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Hot prefix (Elamur summary, Summary 1st paragraph: a small set of "hot" neurons fires for
 * most inputs; Interesting ideas, I1: the most used parts go first).  In a hot-first layer
 * (psffn_permute_hot_first) the neurons [0, n_hot) are listed for every batch without consulting
 * the predictor, which decides only for [n_hot, F).  The list is the ascending union of the two.
 *   n_hot   0 <= n_hot <= F (E_INVALID_ARG otherwise); 0 gives psffn_predict / psffn_layer exactly
 *   logits  as psffn_predict for neurons >= n_hot; the entries of hot neurons are unspecified
 * Where the small-batch predictor runs (fp32 predictors up to 4 tokens; fp16 ones at 1 token, and at
 * 2 tokens up to 1024 ranks) it does not read the Q rows of the hot prefix (F-n_hot rows stream
 * instead of F); the batch predictor computes every logit and forces the prefix into the list.
 * Everything else (arguments, outputs, workspace, errors) is as in psffn_predict / psffn_layer. */
psffn_status psffn_predict_hot(const psffn_predictor* P, int n_hot, const void* x, int B, float logit_thr,
                               int32_t* idx, int32_t* count, float* logits, void* ws, size_t ws_bytes,
                               hipStream_t stream);
psffn_status psffn_layer_hot(const psffn_predictor* P, const psffn_ffn* W, int n_hot, const void* x, int B,
                             float logit_thr, int32_t* idx, int32_t* count, float* logits, float* y, int accumulate,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* One step of a decode stack (the residual update between layers), in one call:
 *   h = fp16(LayerNorm(x))   (gamma 1, beta 0, population variance, eps; as psffn_layernorm_f16)
 *   x += FFN restricted to the predicted neurons of h   (psffn_layer on h with y = x, accumulate)
 * with exactly the outputs of psffn_layernorm_f16 followed by that psffn_layer call.
 *   x    in/out, fp32 [B][d] residual, 16-byte aligned
 *   h    out, fp16 [B][d] (16-byte aligned, not overlapping x): the FFN input
 *   P    fp16 predictor (E_UNSUPPORTED otherwise); the other arguments as psffn_layer.
 * Where the small-batch pipeline runs the layer, the LayerNorm is computed inside the layer's first
 * kernel (no separate launch). */
psffn_status psffn_layer_ln(const psffn_predictor* P, const psffn_ffn* W, float* x, float eps, void* h, int B,
                            float logit_thr, int32_t* idx, int32_t* count, float* logits, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* psffn_layer without a workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The library
 * allocates nothing here either: the workspace is a static device array of
 * PSFFN_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds until the process
 * ends.  The first call on a device looks up that device's copy and clears it with a fill kernel on
 * the given stream.
 *   Arguments, outputs and errors are those of psffn_layer (no hot prefix).  A shape whose
 *   workspace (psffn_workspace_bytes(P, W, B)) exceeds PSFFN_NOALLOC_SCRATCH_BYTES is rejected with
 *   PSFFN_E_WORKSPACE before anything is enqueued.
 *   Every call on one GPU shares that GPU's array, which keeps the last call's contents: calls that
 *   overlap on one GPU (unordered streams, concurrent host threads) race and give undefined outputs;
 *   calls ordered on one stream are independent of each other. */
#define PSFFN_NOALLOC_SCRATCH_BYTES (64u << 20)
psffn_status psffn_layer_noalloc(const psffn_predictor* P, const psffn_ffn* W, const void* x, int B,
                                 float logit_thr, int32_t* idx, int32_t* count, float* logits, float* y,
                                 int accumulate, hipStream_t stream);

/* Offline activation profile (Summary, 2nd paragraph: models are profiled offline):
 * counts[i] = number of the T tokens X [T][d] for which neuron i truly fires -- the ReLU
 * pre-activation W_up[i].x + b_up[i] > 0, or for SwiGLU the gate W_gate[i].x + b_gate[i] > 0.
 * counts: int32 [F], overwritten.  T >= 1. */
psffn_status psffn_profile_counts(const psffn_ffn* W, const void* X, int T, int32_t* counts, hipStream_t stream);

/* Hot-first neuron order (Interesting ideas, I1: the most used parts go first; Summary, 2nd
 * paragraph: the neurons are profiled offline by how often they fire).
 *   counts  int32 [F] fire counts (e.g. from psffn_profile_counts)
 *   perm    out, int32 [F]: perm[k] = original neuron placed at position k, in descending
 *           count order, ties by ascending original index (stable)
 *   src/dst FFN layers (dst names caller-owned buffers of the same shapes and types; the
 *           library writes dst row k = src row perm[k] of every neuron-indexed tensor:
 *           w_up, w_gate, w_dT, their scales, b_up, b_gate; b_down is not neuron-indexed and is
 *           not touched)
 *   psrc/pdst  predictors: pdst Q row k = psrc Q row perm[k], c likewise; A is not
 *           neuron-indexed and is not touched.
 * Either pair may be NULL to permute only the other.  Out-of-place: dst buffers must not
 * overlap src buffers (E_INVALID_ARG otherwise).  Needs no workspace. */
psffn_status psffn_permute_hot_first(const int32_t* counts, int F, int32_t* perm, const psffn_ffn* src,
                                     const psffn_ffn* dst, const psffn_predictor* psrc, const psffn_predictor* pdst,
                                     hipStream_t stream);

/* Decode-stack glue: out_f16[b] = fp16(LayerNorm(x[b])) with gamma 1, beta 0, population
 * variance and the given eps; x is the fp32 residual stream [B][d] (any B >= 1, d % 4 == 0). */
psffn_status psffn_layernorm_f16(const float* x, int B, int d, float eps, void* out_f16, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* psffn_status_str(psffn_status s);

#ifdef __cplusplus
}
#endif

#endif /* PSFFN_H_ */

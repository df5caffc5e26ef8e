// Internal definitions of libpsffn (gfx950 / CDNA4, wave64): storage traits, 16-byte lane
// vectors, dot products, wave reductions, workspace layout and the launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psffn.h"

namespace psffn {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // 4 waves per workgroup
constexpr int kSplitCap = 64;  // max number of k-splits of the down projection (partials buffer)
constexpr int kSplitMinRows = 16;  // min rows per k-split
constexpr int kUDSplitCap = 256;   // max splits of the small-batch fused up/down kernel (partials buffer)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

enum class St : int { F32 = 0, F16 = 1, I4 = 2 };

// ----------------------------------------------------------------------------------------
// elementwise helpers

__device__ __forceinline__ float wave_sum(float v) {
  // xor butterfly: every lane ends with the same, order-fixed sum
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_lane() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
}

// 8 fp16 weights x 8 fp16 activations, fp32 accumulation (products of two halves are exact in fp32)
__device__ __forceinline__ float dot8_f16(uint4 w, uint4 x, float acc) {
  acc = dot2_f16(w.x, x.x, acc);
  acc = dot2_f16(w.y, x.y, acc);
  acc = dot2_f16(w.z, x.z, acc);
  acc = dot2_f16(w.w, x.w, acc);
  return acc;
}

__device__ __forceinline__ float dot4_f32(uint4 w, uint4 x, float acc) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}

// 8 fp16 weights x 8 fp32 values (the predictor's second stage keeps h in fp32)
__device__ __forceinline__ float dot8_f16_f32(uint4 w, float4 h0, float4 h1, float acc) {
  acc = fmaf(h2f(w.x & 0xffff), h0.x, acc);
  acc = fmaf(h2f(w.x >> 16), h0.y, acc);
  acc = fmaf(h2f(w.y & 0xffff), h0.z, acc);
  acc = fmaf(h2f(w.y >> 16), h0.w, acc);
  acc = fmaf(h2f(w.z & 0xffff), h1.x, acc);
  acc = fmaf(h2f(w.z >> 16), h1.y, acc);
  acc = fmaf(h2f(w.w & 0xffff), h1.z, acc);
  acc = fmaf(h2f(w.w >> 16), h1.w, acc);
  return acc;
}

// ---- 4-bit weights.  One 32-bit word holds 8 consecutive elements e0..e7, e_k in bits
// [4k, 4k+4), each a two's-complement nibble.  Decoding trick: (nibble ^ 8) placed in the
// mantissa of the fp16 1024.0 gives 1024 + q + 8 exactly; subtracting 1032 leaves q exactly.
// The pairs come out as (e0,e4), (e1,e5), (e2,e6), (e3,e7); activations are paired the same
// way by pair_x8.
__device__ __forceinline__ half2_t i4_pair(uint32_t w, int shift) {
  uint32_t b = ((w >> shift) & 0x000F000Fu) ^ 0x64086408u;
  half2_t v = __builtin_bit_cast(half2_t, b);
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  return v - off;
}

// 8 fp16 activations x0..x7 -> pairs (x0,x4), (x1,x5), (x2,x6), (x3,x7)
__device__ __forceinline__ uint4 pair_x8(uint4 x) {
  uint4 p;
  p.x = (x.x & 0xffffu) | (x.z << 16);
  p.y = (x.x >> 16) | (x.z & 0xffff0000u);
  p.z = (x.y & 0xffffu) | (x.w << 16);
  p.w = (x.y >> 16) | (x.w & 0xffff0000u);
  return p;
}

// sum_{k<8} q_k * x_k for one word of nibbles and paired activations (exact products)
__device__ __forceinline__ float dot8_i4(uint32_t w, uint4 px, float acc) {
  acc = __builtin_amdgcn_fdot2(i4_pair(w, 0), __builtin_bit_cast(half2_t, px.x), acc, false);
  acc = __builtin_amdgcn_fdot2(i4_pair(w, 4), __builtin_bit_cast(half2_t, px.y), acc, false);
  acc = __builtin_amdgcn_fdot2(i4_pair(w, 8), __builtin_bit_cast(half2_t, px.z), acc, false);
  acc = __builtin_amdgcn_fdot2(i4_pair(w, 12), __builtin_bit_cast(half2_t, px.w), acc, false);
  return acc;
}

// signed nibble k (0..7) of a word as float
__device__ __forceinline__ float i4_elem(uint32_t w, int k) {
  return (float)(((int32_t)(w << (28 - 4 * k))) >> 28);
}

// ----------------------------------------------------------------------------------------
// workspace layout (bytes, every region 256-byte aligned)
//
//   [0, 256)      reserved header
//   mask words    one 32-bit word of active bits per 32 neurons (predictor -> list / fused FFN)
//   scratch       per-call buffers (h, flags, activations, partials); dead between calls
// The layout depends on F only, so the predictor and the FFN of one layer can share one
// workspace.  No region carries state from one call to the next.

constexpr int kMaxD = 262144;

__host__ __device__ inline size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

struct StateLayout {
  size_t masks, scratch;
};

__host__ __device__ inline StateLayout state_layout(int F) {
  StateLayout s;
  s.masks = 256;
  s.scratch = s.masks + round256(4 * (size_t)((F + 31) / 32));
  return s;
}

// Sum over a workgroup of kBlock threads (wave sums, then the wave totals in wave order).
__device__ __forceinline__ float block_sum(float v, float* s_red) {
  v = wave_sum(v);
  __syncthreads();
  if (wave_lane() == 0) s_red[wave_id()] = v;
  __syncthreads();
  float t = 0.f;
  for (int k = 0; k < kBlock / kWave; ++k) t += s_red[k];
  return t;
}

// One LayerNorm row (gamma 1, beta 0, population variance, fp16 result) by a workgroup of kBlock
// threads, the row held in registers: thread t holds float4 j = t + k kBlock (k < K, d % 4 == 0).
// Two block reductions (mean, then the centred sum of squares), then out[j] = 4 halves (uint2;
// global or LDS).  The LayerNorm kernel and the layer call's first kernel both use it, so they give
// the same bits.
// The row's loads (ln_row_load) and the rest (ln_row_finish) are separate so that a caller can
// issue the loads early; ln_row_f16 is the two in a row.
template <int K>
__device__ __forceinline__ void ln_row_load(const float* __restrict__ xrow, int d, float4 (&v)[K]) {
  const float4* xr = reinterpret_cast<const float4*>(xrow);
  const int n4 = d / 4;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = threadIdx.x + k * kBlock;
    v[k] = j < n4 ? xr[j] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int K>
__device__ __forceinline__ void ln_row_finish(const float4 (&v)[K], int d, float eps, float* s_red, uint2* out) {
  const int n4 = d / 4;
  float sm = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) sm += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  const float mean = block_sum(sm, s_red) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (threadIdx.x + k * kBlock < n4) {
      const float a = v[k].x - mean, b = v[k].y - mean, c = v[k].z - mean, e = v[k].w - mean;
      q = fmaf(a, a, q);
      q = fmaf(b, b, q);
      q = fmaf(c, c, q);
      q = fmaf(e, e, q);
    }
  }
  const float var = block_sum(q, s_red) / (float)d;
  const float inv = 1.f / sqrtf(var + eps);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = threadIdx.x + k * kBlock;
    if (j < n4) {
      const half2_t lo = {(_Float16)((v[k].x - mean) * inv), (_Float16)((v[k].y - mean) * inv)};
      const half2_t hi = {(_Float16)((v[k].z - mean) * inv), (_Float16)((v[k].w - mean) * inv)};
      out[j] = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  }
}

template <int K>
__device__ __forceinline__ void ln_row_f16(const float* __restrict__ xrow, int d, float eps, float* s_red,
                                           uint2* out) {
  float4 v[K];
  ln_row_load<K>(xrow, d, v);
  ln_row_finish<K>(v, d, eps, s_red, out);
}

// float4 per thread that ln_row_f16 needs for a row of d (1, 2, 4, 8 or 16; 0 above 16384)
inline int ln_k(int d) {
  const int k = (d / 4 + kBlock - 1) / kBlock;
  return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : 0;
}

// ----------------------------------------------------------------------------------------
// launchers (return hipSuccess or the launch error)

hipError_t launch_pred_h(St st, const void* A, const void* x, int B, int d, int r, float* h, hipStream_t s);
hipError_t launch_pred_logits(St st, const void* Q, const float* c, const float* h, int B, int r, int F, float thr,
                              float* logits, uint8_t* flags, hipStream_t s);
hipError_t launch_flags_from_logits(const float* logits, int B, int F, float thr, uint8_t* flags, hipStream_t s);
hipError_t launch_scatter(const uint8_t* flags, int F, int32_t* idx, int32_t* count, hipStream_t s, int n_hot = 0);
hipError_t launch_up(St st, psffn_act act, const psffn_ffn& W, const void* x, int B, const int32_t* idx,
                     const int32_t* count, float* a, hipStream_t s);
hipError_t launch_down(St st, const psffn_ffn& W, const float* a, int B, const int32_t* idx, const int32_t* count,
                       float* part, hipStream_t s);
hipError_t launch_reduce(const float* part, const int32_t* count, int F, int B, int d, const float* b_down, float* y,
                         int accumulate, hipStream_t s);
hipError_t launch_profile_counts(St st, const psffn_ffn& W, const void* X, int T, int32_t* counts, hipStream_t s);
hipError_t launch_hot_first_perm(const int32_t* counts, int F, int32_t* perm, hipStream_t s);
hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* perm, int F, size_t row_bytes,
                              hipStream_t s);
hipError_t launch_layernorm_f16(const float* x, int B, int d, float eps, void* out, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// small-batch pipeline (batch <= kFusedMaxBatch): predictor in two kernels (h, then logits with
// the ordered compaction), FFN in two kernels (up rows, then down tiles with the reduction).
// They return hipErrorNotSupported when the shape is outside what they handle, and the caller
// takes the generic kernels.
constexpr int kFusedMaxBatch = 4;
// n_hot: neurons [0, n_hot) are listed whatever their logits (0 <= n_hot <= F)
hipError_t launch_predict_fused(St st, const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx,
                                int32_t* count, float* logits, void* ws, hipStream_t s, int n_hot = 0);
hipError_t launch_ffn_fused(St st, const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count,
                            float* y, int accumulate, void* ws, hipStream_t s);
// the small-batch FFN from the mask words of a predictor call in the same workspace (the list and its
// length are ordered inside the fused kernel and written to idx/count, as in launch_layer_fused)
bool ffn_fused_scan_fits(const psffn_ffn& W, int B);  // launch_ffn_fused_scan can run this shape
hipError_t launch_ffn_fused_scan(St st, const psffn_ffn& W, const void* x, int B, int32_t* idx, int32_t* count,
                                 float* y, int accumulate, void* ws, hipStream_t s, int n_hot);
// LayerNorm folded into the layer call (stack step): xres = the fp32 residual (the input of the
// LayerNorm), hout = its fp16 LayerNorm output, written by the call and read by its FFN
struct LnArgs {
  const float* xres = nullptr;
  float eps = 0.f;
  _Float16* hout = nullptr;
};
hipError_t launch_layer_fused(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                              int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                              hipStream_t s, int n_hot = 0, const LnArgs& ln = LnArgs{});

// k_h alone at one token (fp16 predictor), with the stack step's LayerNorm when ln.xres is set; it
// also zeroes the nzero words at zero and the nzero2 words at zero2 (for the launch after it, which
// ORs bits and counts into them)
hipError_t launch_h_f16_b1(const psffn_predictor& P, const void* x, float* h, const LnArgs& ln, hipStream_t s,
                           uint32_t* zero, int nzero, uint32_t* zero2, int nzero2);

// streamed one-token pipeline (stream.hip; fp16 predictor, fp16 or 4-bit ReLU weights): the up rows
// ride on the logits kernel, the down projection sums its split partials itself.  Scratch after the
// mask words: stream_scratch bytes.  NotSupported outside the shapes the *_fits calls accept.
size_t stream_scratch(int r, int F, int d);
bool stream_ffn_fits(const psffn_ffn& W, int B);     // one token, fp16 ReLU weights: k_up1 + k_dn
bool stream_ffn_i4_fits(const psffn_ffn& W, int B);  // one token, 4-bit ReLU weights: k_up1_i4 + k_dn
// h = A x at one token by k_h1 (fp16 predictor, rows of A up to 12288): the bits of k_h
hipError_t launch_h1(const psffn_predictor& P, const void* x, float* h, hipStream_t s);
bool stream_layer_fits(const psffn_predictor& P, const psffn_ffn& W, int B, bool ln);
hipError_t launch_ffn_stream(const psffn_ffn& W, const void* x, const int32_t* idx, const int32_t* count, float* y,
                             int accumulate, void* ws, hipStream_t s);
hipError_t launch_layer_stream(const psffn_predictor& P, const psffn_ffn& W, const void* x, float thr, int32_t* idx,
                               int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s,
                               int n_hot, const LnArgs& ln);

// batch pipeline (2 <= B <= 32, fp16 predictor, fp16 or 4-bit FFN weights) on MFMA tiles; the
// same NotSupported convention.  Above kFusedMaxBatch tokens it is the only pipeline; from 2 to
// kFusedMaxBatch tokens the calls choose per stage (pred_on_batch / ffn_on_batch in api.hip).
bool batch_supported_pred(const psffn_predictor& P, int B);
bool batch_supported_ffn(const psffn_ffn& W, int B);
size_t batch_scratch_bytes(int B, int d, int r, int F, psffn_dtype wdt, psffn_act act, bool pred, bool ffn);
hipError_t launch_predict_batch(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx,
                                int32_t* count, float* logits, void* ws, hipStream_t s, int n_hot = 0);
// the batch predictor's kernels up to its mask words (in the workspace's mask region), no list
hipError_t launch_predict_batch_masks(const psffn_predictor& P, const void* x, int B, float thr, float* logits,
                                      void* ws, hipStream_t s);
hipError_t launch_ffn_batch(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count,
                            float* y, int accumulate, void* ws, hipStream_t s);
hipError_t launch_layer_batch(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                              int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                              hipStream_t s, int n_hot = 0);

}  // namespace psffn

namespace psffn {

// ----------------------------------------------------------------------------------------
// One lane's 16-byte slice of a weight row against the matching activations of one token.
//   F32: 4 elements, F16: 8 elements, I4: 32 elements (4 words of nibbles, one group scale).
// `e` is the element index of the slice's first element; x points at the token's row.

template <St WT> struct Tr;
template <> struct Tr<St::F32> { static constexpr int EPL = 4; static constexpr int ESZ = 4; };
template <> struct Tr<St::F16> { static constexpr int EPL = 8; static constexpr int ESZ = 2; };
template <> struct Tr<St::I4> { static constexpr int EPL = 32; static constexpr int ESZ = 0; };

// bytes of one weight row of d elements
template <St WT> __host__ __device__ inline size_t row_bytes(int d) {
  return WT == St::F32 ? (size_t)d * 4 : (WT == St::F16 ? (size_t)d * 2 : (size_t)d / 2);
}

template <St WT>
__device__ __forceinline__ float dot16(uint4 w, const void* __restrict__ x, int e, float scale, float acc) {
  if constexpr (WT == St::F32) {
    uint4 xv = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + e);
    return dot4_f32(w, xv, acc);
  } else if constexpr (WT == St::F16) {
    uint4 xv = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(x) + e);
    return dot8_f16(w, xv, acc);
  } else {
    const uint4* xp = reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(x) + e);
    float part = 0.f;
    part = dot8_i4(w.x, pair_x8(xp[0]), part);
    part = dot8_i4(w.y, pair_x8(xp[1]), part);
    part = dot8_i4(w.z, pair_x8(xp[2]), part);
    part = dot8_i4(w.w, pair_x8(xp[3]), part);
    return fmaf(scale, part, acc);
  }
}

}  // namespace psffn

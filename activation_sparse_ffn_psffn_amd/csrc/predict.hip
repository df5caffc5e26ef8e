// Predictor kernels: h = A x (fp32), logits l = Q h + c with the strict threshold test, and the
// ordered compaction of the active neurons into an ascending index list.
//
// The pages ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur
// Research summary, Summary 2nd paragraph) only say a lightweight per-layer predictor guesses
// which neurons fire; the low-rank linear form and the logit threshold are the readings stated in
// include/psffn.h.
#include "common.h"

namespace psffn {

// h[b][j] = sum_k A[j][k] x[b][k] for tokens b0..b0+nb-1: one wave per row j of A, 16-byte
// coalesced loads along the row, fp32 accumulation, order-fixed wave reduction.
template <St PT, int NB>
__global__ __launch_bounds__(kBlock) void k_pred_h(const void* __restrict__ A, const void* __restrict__ x, int b0,
                                                   int nb, int d, int r, float* __restrict__ h) {
  const int j = blockIdx.x * (kBlock / kWave) + wave_id();
  if (j >= r) return;
  const int lane = wave_lane();
  constexpr int EPL = Tr<PT>::EPL;
  const char* arow = reinterpret_cast<const char*>(A) + (size_t)j * row_bytes<PT>(d);
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  for (int e = lane * EPL; e < d; e += kWave * EPL) {
    uint4 w = *reinterpret_cast<const uint4*>(arow + (size_t)e * Tr<PT>::ESZ);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < nb) {
        const char* xr = reinterpret_cast<const char*>(x) + (size_t)(b0 + b) * d * Tr<PT>::ESZ;
        acc[b] = dot16<PT>(w, xr, e, 1.f, acc[b]);
      }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float s = wave_sum(acc[b]);
    if (lane == 0 && b < nb) h[(size_t)(b0 + b) * r + j] = s;
  }
}

// logits and union flags: 64 neurons per workgroup (16 per wave).  h stays fp32.
// flags[i] = (first ? 0 : flags[i]) | (exists b: l_b,i > thr)
template <St PT, int NB>
__global__ __launch_bounds__(kBlock) void k_pred_logits(const void* __restrict__ Q, const float* __restrict__ c,
                                                        const float* __restrict__ h, int b0, int nb, int r, int F,
                                                        float thr, float* __restrict__ logits,
                                                        uint8_t* __restrict__ flags, int first) {
  const int lane = wave_lane();
  constexpr int EPL = Tr<PT>::EPL;
  for (int q = 0; q < 16; ++q) {
    const int i = blockIdx.x * 64 + wave_id() * 16 + q;
    if (i >= F) break;
    const char* qrow = reinterpret_cast<const char*>(Q) + (size_t)i * row_bytes<PT>(r);
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    for (int e = lane * EPL; e < r; e += kWave * EPL) {
      uint4 w = *reinterpret_cast<const uint4*>(qrow + (size_t)e * Tr<PT>::ESZ);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < nb) {
          const float* hb = h + (size_t)(b0 + b) * r + e;
          if constexpr (PT == St::F32) {
            acc[b] = dot4_f32(w, *reinterpret_cast<const uint4*>(hb), acc[b]);
          } else {
            acc[b] = dot8_f16_f32(w, *reinterpret_cast<const float4*>(hb), *reinterpret_cast<const float4*>(hb + 4),
                                  acc[b]);
          }
        }
    }
    bool on = false;
    const float ci = c[i];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float l = wave_sum(acc[b]) + ci;
      if (b < nb) {
        on |= l > thr;
        if (logits && lane == 0) logits[(size_t)(b0 + b) * F + i] = l;
      }
    }
    if (lane == 0) {
      uint8_t prev = first ? 0 : flags[i];
      flags[i] = (uint8_t)(prev | (on ? 1 : 0));
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_flags_from_logits(const float* __restrict__ logits, int B, int F,
                                                              float thr, uint8_t* __restrict__ flags) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= F) return;
  bool on = false;
  for (int b = 0; b < B; ++b) on |= logits[(size_t)b * F + i] > thr;
  flags[i] = on ? 1 : 0;
}

// Ordered compaction: chunk c (256 neurons) counts the active flags of all earlier chunks, then
// each wave ranks its lanes with ballot + mbcnt.  The last chunk writes the total count.
__global__ __launch_bounds__(kBlock) void k_scatter(const uint8_t* __restrict__ flags, int F, int n_hot,
                                                    int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ int s_red[kBlock / kWave];
  __shared__ int s_wc[kBlock / kWave];
  const int c = blockIdx.x;
  const int lane = wave_lane(), wv = wave_id();
  int pre = 0;
  const int nbytes = c * kBlock;  // multiple of 4; flags region is 4-byte aligned
  const uint32_t* f4 = reinterpret_cast<const uint32_t*>(flags);
  for (int w = threadIdx.x; w < nbytes / 4; w += kBlock) {
    uint32_t v = f4[w];
#pragma unroll
    for (int k = 0; k < 4; ++k) pre += (int)(((v >> (8 * k)) & 1u) | (uint32_t)(4 * w + k < n_hot));
  }
  float ps = wave_sum((float)pre);  // exact: counts < 2^24
  if (lane == 0) s_red[wv] = (int)ps;
  const int i = c * kBlock + threadIdx.x;
  const bool on = i < F && (i < n_hot || flags[i] != 0);
  const unsigned long long bal = __ballot(on);
  const int rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
  if (lane == 0) s_wc[wv] = __popcll(bal);
  __syncthreads();
  int base = 0, wpre = 0, tot = 0;
  for (int k = 0; k < kBlock / kWave; ++k) {
    base += s_red[k];
    if (k < wv) wpre += s_wc[k];
    tot += s_wc[k];
  }
  if (on) idx[base + wpre + rank] = i;
  if (c == (int)gridDim.x - 1 && threadIdx.x == 0) *count = base + tot;
}

// ----------------------------------------------------------------------------------------

template <St PT>
static hipError_t pred_h_t(const void* A, const void* x, int B, int d, int r, float* h, hipStream_t s) {
  dim3 grid((r + 3) / 4);
  for (int b0 = 0; b0 < B; b0 += 8) {
    int nb = B - b0 < 8 ? B - b0 : 8;
    if (nb == 1)
      k_pred_h<PT, 1><<<grid, kBlock, 0, s>>>(A, x, b0, nb, d, r, h);
    else if (nb <= 4)
      k_pred_h<PT, 4><<<grid, kBlock, 0, s>>>(A, x, b0, nb, d, r, h);
    else
      k_pred_h<PT, 8><<<grid, kBlock, 0, s>>>(A, x, b0, nb, d, r, h);
  }
  return hipGetLastError();
}

hipError_t launch_pred_h(St st, const void* A, const void* x, int B, int d, int r, float* h, hipStream_t s) {
  return st == St::F32 ? pred_h_t<St::F32>(A, x, B, d, r, h, s) : pred_h_t<St::F16>(A, x, B, d, r, h, s);
}

template <St PT>
static hipError_t pred_logits_t(const void* Q, const float* c, const float* h, int B, int r, int F, float thr,
                                float* logits, uint8_t* flags, hipStream_t s) {
  dim3 grid((F + 63) / 64);
  for (int b0 = 0; b0 < B; b0 += 8) {
    int nb = B - b0 < 8 ? B - b0 : 8;
    int first = b0 == 0;
    if (nb == 1)
      k_pred_logits<PT, 1><<<grid, kBlock, 0, s>>>(Q, c, h, b0, nb, r, F, thr, logits, flags, first);
    else if (nb <= 4)
      k_pred_logits<PT, 4><<<grid, kBlock, 0, s>>>(Q, c, h, b0, nb, r, F, thr, logits, flags, first);
    else
      k_pred_logits<PT, 8><<<grid, kBlock, 0, s>>>(Q, c, h, b0, nb, r, F, thr, logits, flags, first);
  }
  return hipGetLastError();
}

hipError_t launch_pred_logits(St st, const void* Q, const float* c, const float* h, int B, int r, int F, float thr,
                              float* logits, uint8_t* flags, hipStream_t s) {
  return st == St::F32 ? pred_logits_t<St::F32>(Q, c, h, B, r, F, thr, logits, flags, s)
                       : pred_logits_t<St::F16>(Q, c, h, B, r, F, thr, logits, flags, s);
}

hipError_t launch_flags_from_logits(const float* logits, int B, int F, float thr, uint8_t* flags, hipStream_t s) {
  k_flags_from_logits<<<(F + kBlock - 1) / kBlock, kBlock, 0, s>>>(logits, B, F, thr, flags);
  return hipGetLastError();
}

hipError_t launch_scatter(const uint8_t* flags, int F, int32_t* idx, int32_t* count, hipStream_t s, int n_hot) {
  k_scatter<<<(F + kBlock - 1) / kBlock, kBlock, 0, s>>>(flags, F, n_hot, idx, count);
  return hipGetLastError();
}

}  // namespace psffn

// Sparse FFN kernels over a neuron list ("PowerInfer: Fast Large Language Model Serving with a
// Consumer-grade GPU", Elamur Research summary, Summary 2nd paragraph: compute only the predicted
// neurons and skip the rest; Interesting ideas I4: act on whole weight rows, no sparse format).
//
//   up:     a[k][b] = act(W_up[idx[k]] . x_b (+ gate branch))      one wave per listed row
//   down:   part[s][b][cols] = sum_{k in split s} a[k][b] W_dT[idx[k]][cols]
//   reduce: y[b][j] (+)= b_down[j] + sum_{s ascending} part[s][b][j]
// The split of the list into k-ranges is a fixed function of count, so y is bit-reproducible
// (no floating-point atomics anywhere).
#include "common.h"

namespace psffn {

__device__ __forceinline__ int clamp_count(const int32_t* count, int F) {
  int n = *count;
  return n < 0 ? 0 : (n > F ? F : n);
}

// rows per k-split and number of splits for a list of n neurons (n > 0)
__device__ __forceinline__ void split_shape(int n, int& ks, int& S) {
  ks = (n + kSplitCap - 1) / kSplitCap;
  if (ks < kSplitMinRows) ks = kSplitMinRows;
  S = n > 0 ? (n + ks - 1) / ks : 0;
}

template <St WT>
__device__ __forceinline__ float row_scale(const void* s, int i, int d, int e) {
  if constexpr (WT == St::I4) {
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(s) + (size_t)i * (d / 128) + e / 128;
    return h2f(*sc);
  } else {
    return 1.f;
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

// Up (and gate) row-gather GEMV for tokens b0..b0+nb-1.  a layout: [F][B].
template <St WT, psffn_act ACT, int NB>
__global__ __launch_bounds__(kBlock) void k_up(const void* __restrict__ w_up, const void* __restrict__ s_up,
                                               const void* __restrict__ w_gate, const void* __restrict__ s_gate,
                                               const float* __restrict__ b_up, const float* __restrict__ b_gate,
                                               const void* __restrict__ x, int b0, int nb, int B, int d, int F,
                                               const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                               float* __restrict__ a) {
  const int n = clamp_count(count, F);
  const int lane = wave_lane();
  const int nw = gridDim.x * (kBlock / kWave);
  constexpr int EPL = Tr<WT>::EPL;
  constexpr int XSZ = WT == St::F32 ? 4 : 2;
  for (int k = blockIdx.x * (kBlock / kWave) + wave_id(); k < n; k += nw) {
    const int i = idx[k];
    const bool valid = (unsigned)i < (unsigned)F;
    float u[NB], g[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) u[b] = g[b] = 0.f;
    if (valid) {
      const char* urow = reinterpret_cast<const char*>(w_up) + (size_t)i * row_bytes<WT>(d);
      const char* grow = ACT == PSFFN_SWIGLU ? reinterpret_cast<const char*>(w_gate) + (size_t)i * row_bytes<WT>(d) : nullptr;
      for (int e = lane * EPL; e < d; e += kWave * EPL) {
        const size_t boff = WT == St::I4 ? (size_t)e / 2 : (size_t)e * Tr<WT>::ESZ;
        uint4 wu = *reinterpret_cast<const uint4*>(urow + boff);
        float su = row_scale<WT>(s_up, i, d, e);
        uint4 wg;
        float sg = 1.f;
        if constexpr (ACT == PSFFN_SWIGLU) {
          wg = *reinterpret_cast<const uint4*>(grow + boff);
          sg = row_scale<WT>(s_gate, i, d, e);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < nb) {
            const char* xr = reinterpret_cast<const char*>(x) + (size_t)(b0 + b) * d * XSZ;
            u[b] = dot16<WT>(wu, xr, e, su, u[b]);
            if constexpr (ACT == PSFFN_SWIGLU) g[b] = dot16<WT>(wg, xr, e, sg, g[b]);
          }
      }
    }
    const float bu = (valid && b_up) ? b_up[i] : 0.f;
    const float bg = (valid && b_gate) ? b_gate[i] : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float uu = wave_sum(u[b]) + bu;
      float av;
      if constexpr (ACT == PSFFN_SWIGLU) {
        float gg = wave_sum(g[b]) + bg;
        av = silu(gg) * uu;
      } else {
        av = uu > 0.f ? uu : 0.f;
      }
      if (!valid) av = 0.f;
      if (lane == 0 && b < nb) a[(size_t)k * B + b0 + b] = av;
    }
  }
}

// Down projection into split partials.  Workgroup (t, s): column tile t (each lane owns CPL
// consecutive columns), k-split s; its 4 waves take the split's rows round-robin and are summed in
// wave order through LDS.  part layout: [kSplitCap][B][d].
template <St WT> struct Down;
template <> struct Down<St::F32> { static constexpr int CPL = 4; };
template <> struct Down<St::F16> { static constexpr int CPL = 8; };
template <> struct Down<St::I4> { static constexpr int CPL = 16; };

template <St WT, int NB>
__global__ __launch_bounds__(kBlock) void k_down(const void* __restrict__ w_dT, const void* __restrict__ s_dT,
                                                 const float* __restrict__ a, int b0, int nb, int B, int d, int F,
                                                 const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                                 float* __restrict__ part) {
  constexpr int CPL = Down<WT>::CPL;
  constexpr int TW = kWave * CPL;
  __shared__ float s_acc[NB * TW];
  const int n = clamp_count(count, F);
  int ks, S;
  split_shape(n, ks, S);
  const int s = blockIdx.y;
  if (s >= S) return;
  const int lane = wave_lane(), wv = wave_id();
  const int col0 = blockIdx.x * TW + lane * CPL;
  const bool live = col0 < d;
  const int k_lo = s * ks;
  const int k_hi = min(n, k_lo + ks);
  float acc[NB][CPL];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[b][e] = 0.f;
  if (live) {
    for (int k = k_lo + wv; k < k_hi; k += kBlock / kWave) {
      const int i = idx[k];
      if ((unsigned)i >= (unsigned)F) continue;
      float w[CPL];
      if constexpr (WT == St::F32) {
        uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(w_dT) + (size_t)i * d + col0);
        w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y); w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
      } else if constexpr (WT == St::F16) {
        uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(w_dT) + (size_t)i * d + col0);
        w[0] = h2f(v.x & 0xffff); w[1] = h2f(v.x >> 16); w[2] = h2f(v.y & 0xffff); w[3] = h2f(v.y >> 16);
        w[4] = h2f(v.z & 0xffff); w[5] = h2f(v.z >> 16); w[6] = h2f(v.w & 0xffff); w[7] = h2f(v.w >> 16);
      } else {
        uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(w_dT) + (size_t)i * (d / 2) + col0 / 2);
        const float sc = row_scale<WT>(s_dT, i, d, col0);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = i4_elem(v.x, e) * sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[8 + e] = i4_elem(v.y, e) * sc;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < nb) {
          const float ab = a[(size_t)k * B + b0 + b];
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[b][e] = fmaf(ab, w[e], acc[b][e]);
        }
    }
  }
  // fixed-order combination of the 4 waves: wave 0 stores, waves 1..3 add in turn, wave 3 writes out
  for (int step = 0; step < kBlock / kWave; ++step) {
    if (wv == step) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int at = b * TW + lane * CPL + e;
          float v = step == 0 ? acc[b][e] : s_acc[at] + acc[b][e];
          if (step < kBlock / kWave - 1) {
            s_acc[at] = v;
          } else if (live && b < nb && col0 + e < d) {
            part[((size_t)s * B + b0 + b) * d + col0 + e] = v;
          }
        }
    }
    __syncthreads();
  }
}

// y[b][j] = (accumulate ? y[b][j] : 0) + (b_down[j] + sum_{s < S} part[s][b][j])
__global__ __launch_bounds__(kBlock) void k_reduce(const float* __restrict__ part, const int32_t* __restrict__ count,
                                                   int F, int B, int d, const float* __restrict__ b_down,
                                                   float* __restrict__ y, int accumulate) {
  const int n = clamp_count(count, F);
  int ks, S;
  split_shape(n, ks, S);
  const size_t t = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (size_t)B * d) return;
  const int b = (int)(t / d), j = (int)(t % d);
  float v = b_down ? b_down[j] : 0.f;
  for (int s = 0; s < S; ++s) v += part[((size_t)s * B + b) * d + j];
  y[t] = accumulate ? y[t] + v : v;
}

// ----------------------------------------------------------------------------------------

static int up_grid(int F) {
  int g = (F + 3) / 4;
  return g > 4096 ? 4096 : (g < 1 ? 1 : g);
}

template <St WT, psffn_act ACT>
static hipError_t up_t(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count, float* a,
                       hipStream_t s) {
  dim3 grid(up_grid(W.F));
  for (int b0 = 0; b0 < B; b0 += 8) {
    int nb = B - b0 < 8 ? B - b0 : 8;
#define PSFFN_UP(NBV)                                                                                           \
  k_up<WT, ACT, NBV><<<grid, kBlock, 0, s>>>(W.w_up, W.s_up, W.w_gate, W.s_gate, W.b_up, W.b_gate, x, b0, nb, B, \
                                             W.d, W.F, idx, count, a)
    if (nb == 1)
      PSFFN_UP(1);
    else if (nb <= 4)
      PSFFN_UP(4);
    else
      PSFFN_UP(8);
#undef PSFFN_UP
  }
  return hipGetLastError();
}

hipError_t launch_up(St st, psffn_act act, const psffn_ffn& W, const void* x, int B, const int32_t* idx,
                     const int32_t* count, float* a, hipStream_t s) {
  if (act == PSFFN_RELU) {
    if (st == St::F32) return up_t<St::F32, PSFFN_RELU>(W, x, B, idx, count, a, s);
    if (st == St::F16) return up_t<St::F16, PSFFN_RELU>(W, x, B, idx, count, a, s);
    return up_t<St::I4, PSFFN_RELU>(W, x, B, idx, count, a, s);
  }
  if (st == St::F32) return up_t<St::F32, PSFFN_SWIGLU>(W, x, B, idx, count, a, s);
  if (st == St::F16) return up_t<St::F16, PSFFN_SWIGLU>(W, x, B, idx, count, a, s);
  return up_t<St::I4, PSFFN_SWIGLU>(W, x, B, idx, count, a, s);
}

template <St WT>
static hipError_t down_t(const psffn_ffn& W, const float* a, int B, const int32_t* idx, const int32_t* count,
                         float* part, hipStream_t s) {
  constexpr int TW = kWave * Down<WT>::CPL;
  dim3 grid((W.d + TW - 1) / TW, kSplitCap);
  for (int b0 = 0; b0 < B; b0 += 8) {
    int nb = B - b0 < 8 ? B - b0 : 8;
    if (nb == 1)
      k_down<WT, 1><<<grid, kBlock, 0, s>>>(W.w_dT, W.s_dT, a, b0, nb, B, W.d, W.F, idx, count, part);
    else if (nb <= 4)
      k_down<WT, 4><<<grid, kBlock, 0, s>>>(W.w_dT, W.s_dT, a, b0, nb, B, W.d, W.F, idx, count, part);
    else
      k_down<WT, 8><<<grid, kBlock, 0, s>>>(W.w_dT, W.s_dT, a, b0, nb, B, W.d, W.F, idx, count, part);
  }
  return hipGetLastError();
}

hipError_t launch_down(St st, const psffn_ffn& W, const float* a, int B, const int32_t* idx, const int32_t* count,
                       float* part, hipStream_t s) {
  if (st == St::F32) return down_t<St::F32>(W, a, B, idx, count, part, s);
  if (st == St::F16) return down_t<St::F16>(W, a, B, idx, count, part, s);
  return down_t<St::I4>(W, a, B, idx, count, part, s);
}

hipError_t launch_reduce(const float* part, const int32_t* count, int F, int B, int d, const float* b_down, float* y,
                         int accumulate, hipStream_t s) {
  size_t n = (size_t)B * d;
  k_reduce<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, s>>>(part, count, F, B, d, b_down, y, accumulate);
  return hipGetLastError();
}

}  // namespace psffn

// Off-path and glue kernels: the offline fire-count profile, the hot-first order and row
// gather, the decode-stack layer norm, and a zero fill for workspaces.
#include "common.h"

namespace psffn {

// counts[i] = #{t < T : pre-activation of neuron i on token t > 0}
// ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur Research
// summary, Summary 2nd paragraph: the system profiles models offline).  The deciding branch is
// up for ReLU, gate for SwiGLU.  One wave per neuron; tokens come from L2.
template <St WT>
__global__ __launch_bounds__(kBlock) void k_profile_counts(const void* __restrict__ w, const void* __restrict__ sc,
                                                           const float* __restrict__ bias,
                                                           const void* __restrict__ X, int T, int d, int F,
                                                           int32_t* __restrict__ counts) {
  const int lane = wave_lane();
  const int nw = gridDim.x * (kBlock / kWave);
  constexpr int EPL = Tr<WT>::EPL;
  constexpr int XSZ = WT == St::F32 ? 4 : 2;
  for (int i = blockIdx.x * (kBlock / kWave) + wave_id(); i < F; i += nw) {
    const char* row = reinterpret_cast<const char*>(w) + (size_t)i * row_bytes<WT>(d);
    const float bi = bias ? bias[i] : 0.f;
    int n = 0;
    for (int t = 0; t < T; ++t) {
      const char* xr = reinterpret_cast<const char*>(X) + (size_t)t * d * XSZ;
      float acc = 0.f;
      for (int e = lane * EPL; e < d; e += kWave * EPL) {
        const size_t boff = WT == St::I4 ? (size_t)e / 2 : (size_t)e * Tr<WT>::ESZ;
        uint4 wv = *reinterpret_cast<const uint4*>(row + boff);
        float s = 1.f;
        if constexpr (WT == St::I4) s = h2f(reinterpret_cast<const uint16_t*>(sc)[(size_t)i * (d / 128) + e / 128]);
        acc = dot16<WT>(wv, xr, e, s, acc);
      }
      n += (wave_sum(acc) + bi) > 0.f ? 1 : 0;
    }
    if (lane == 0) counts[i] = n;
  }
}

// Hot-first order (Interesting ideas, I1: the most used parts first).  The position of neuron i
// is #{j : c_j > c_i} + #{j < i : c_j == c_i} -- a stable descending sort, computed by counting.
__global__ __launch_bounds__(kBlock) void k_hot_first_perm(const int32_t* __restrict__ counts, int F,
                                                           int32_t* __restrict__ perm) {
  __shared__ int32_t s_c[kBlock];
  const int i = blockIdx.x * kBlock + threadIdx.x;
  const int32_t ci = i < F ? counts[i] : 0;
  int rank = 0;
  for (int j0 = 0; j0 < F; j0 += kBlock) {
    const int j = j0 + threadIdx.x;
    s_c[threadIdx.x] = j < F ? counts[j] : 0;
    __syncthreads();
    const int m = F - j0 < kBlock ? F - j0 : kBlock;
    for (int q = 0; q < m; ++q) {
      const int32_t cj = s_c[q];
      rank += (cj > ci) || (cj == ci && j0 + q < i);
    }
    __syncthreads();
  }
  if (i < F) perm[rank] = i;
}

// dst row k = src row perm[k]; one workgroup per destination row (grid-stride), copy unit U bytes
template <typename U>
__global__ __launch_bounds__(kBlock) void k_gather_rows(const U* __restrict__ src, U* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int F, size_t units) {
  for (int k = blockIdx.x; k < F; k += gridDim.x) {
    const int p = perm[k];
    if ((unsigned)p >= (unsigned)F) continue;
    const U* s = src + (size_t)p * units;
    U* t = dst + (size_t)k * units;
    for (size_t u = threadIdx.x; u < units; u += kBlock) t[u] = s[u];
  }
}

// out[b] = fp16(LayerNorm(x[b])), gamma 1, beta 0, population variance, two passes (mean, then
// the mean of squared deviations).  One workgroup per token.
__global__ __launch_bounds__(kBlock) void k_layernorm_f16(const float* __restrict__ x, int d, float eps,
                                                          _Float16* __restrict__ out) {
  __shared__ float s_red[kBlock / kWave];
  const float* xr = x + (size_t)blockIdx.x * d;
  _Float16* o = out + (size_t)blockIdx.x * d;
  float s = 0.f;
  for (int k = threadIdx.x; k < d; k += kBlock) s += xr[k];
  const float mean = block_sum(s, s_red) / (float)d;
  float q = 0.f;
  for (int k = threadIdx.x; k < d; k += kBlock) {
    const float t = xr[k] - mean;
    q = fmaf(t, t, q);
  }
  const float var = block_sum(q, s_red) / (float)d;
  const float inv = 1.f / sqrtf(var + eps);
  for (int k = threadIdx.x; k < d; k += kBlock) o[k] = (_Float16)((xr[k] - mean) * inv);
}

// Same result definition, the row held in registers: every load of the row is issued at once
// (K float4 per thread), then two block reductions (mean, then the centred sum of squares) on the
// registers and one fp16 store pass.
template <int K>
__global__ __launch_bounds__(kBlock) void k_layernorm_f16_reg(const float* __restrict__ x, int d, float eps,
                                                              _Float16* __restrict__ out) {
  __shared__ float s_red[kBlock / kWave];
  ln_row_f16<K>(x + (size_t)blockIdx.x * d, d, eps, s_red, reinterpret_cast<uint2*>(out + (size_t)blockIdx.x * d));
}

__global__ __launch_bounds__(kBlock) void k_fill_zero(uint4* __restrict__ p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

// ----------------------------------------------------------------------------------------

hipError_t launch_profile_counts(St st, const psffn_ffn& W, const void* X, int T, int32_t* counts, hipStream_t s) {
  const bool relu = W.act == PSFFN_RELU;
  const void* w = relu ? W.w_up : W.w_gate;
  const void* sc = relu ? W.s_up : W.s_gate;
  const float* bias = relu ? W.b_up : W.b_gate;
  int grid = (W.F + 3) / 4;
  if (grid > 4096) grid = 4096;
  if (st == St::F32)
    k_profile_counts<St::F32><<<grid, kBlock, 0, s>>>(w, sc, bias, X, T, W.d, W.F, counts);
  else if (st == St::F16)
    k_profile_counts<St::F16><<<grid, kBlock, 0, s>>>(w, sc, bias, X, T, W.d, W.F, counts);
  else
    k_profile_counts<St::I4><<<grid, kBlock, 0, s>>>(w, sc, bias, X, T, W.d, W.F, counts);
  return hipGetLastError();
}

hipError_t launch_hot_first_perm(const int32_t* counts, int F, int32_t* perm, hipStream_t s) {
  k_hot_first_perm<<<(F + kBlock - 1) / kBlock, kBlock, 0, s>>>(counts, F, perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* perm, int F, size_t row_bytes,
                              hipStream_t s) {
  int grid = F < 8192 ? F : 8192;
  if (grid < 1) return hipSuccess;
  if (row_bytes % 16 == 0)
    k_gather_rows<uint4><<<grid, kBlock, 0, s>>>((const uint4*)src, (uint4*)dst, perm, F, row_bytes / 16);
  else if (row_bytes % 4 == 0)
    k_gather_rows<uint32_t><<<grid, kBlock, 0, s>>>((const uint32_t*)src, (uint32_t*)dst, perm, F, row_bytes / 4);
  else if (row_bytes % 2 == 0)
    k_gather_rows<uint16_t><<<grid, kBlock, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, perm, F, row_bytes / 2);
  else
    k_gather_rows<uint8_t><<<grid, kBlock, 0, s>>>((const uint8_t*)src, (uint8_t*)dst, perm, F, row_bytes);
  return hipGetLastError();
}

hipError_t launch_layernorm_f16(const float* x, int B, int d, float eps, void* out, hipStream_t s) {
  _Float16* o = reinterpret_cast<_Float16*>(out);
  const int k = (d / 4 + kBlock - 1) / kBlock;  // float4 per thread
  const bool vec = d % 4 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)out & 7) == 0;
  if (!vec) k_layernorm_f16<<<B, kBlock, 0, s>>>(x, d, eps, o);
  else if (k <= 1) k_layernorm_f16_reg<1><<<B, kBlock, 0, s>>>(x, d, eps, o);
  else if (k <= 2) k_layernorm_f16_reg<2><<<B, kBlock, 0, s>>>(x, d, eps, o);
  else if (k <= 4) k_layernorm_f16_reg<4><<<B, kBlock, 0, s>>>(x, d, eps, o);
  else if (k <= 8) k_layernorm_f16_reg<8><<<B, kBlock, 0, s>>>(x, d, eps, o);
  else if (k <= 16) k_layernorm_f16_reg<16><<<B, kBlock, 0, s>>>(x, d, eps, o);
  else k_layernorm_f16<<<B, kBlock, 0, s>>>(x, d, eps, o);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t g = (n16 + kBlock - 1) / kBlock;
  k_fill_zero<<<(unsigned)(g > 2048 ? 2048 : g), kBlock, 0, s>>>(reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace psffn

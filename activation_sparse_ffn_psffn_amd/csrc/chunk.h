// The predictor's second stage for one chunk of neurons, shared by the logits kernel of the
// small-batch pipeline (fused.hip k_q) and the streamed batch-1 layer (stream.hip k_qu), so that
// both compute every logit with the same arithmetic and give the same bits.
//
// Method ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur
// Research summary, Summary 2nd paragraph): a per-layer predictor decides which neurons fire.
// Here it is the low-rank form l_i = Q_i . h + c_i with h = A x in fp32, and neuron i is kept when
// l_i > thr for some token of the batch.
#pragma once

#include "common.h"

namespace psffn {

// read through this block when a lane has nothing to load, so every load stays unconditional
static __device__ uint4 q_zero16[1] = {{0u, 0u, 0u, 0u}};  // never written

// Q rows are read once per call: non-temporal loads, so that they do not push the reused lines (h,
// the mask words, the kernels' code) out of L2; each load takes whole lines in one instruction
typedef unsigned int q_u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 q_ld16z(const void* p, bool ok) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                       reinterpret_cast<const q_u32x4v*>(ok ? p : static_cast<const void*>(q_zero16))));
}

// Chunk q of 4*RPW neurons, RPW per wave of a kBlock-thread workgroup.  ILV = 0 (contiguous): bit k
// of the chunk is neuron q*4*RPW + k.  ILV > 0 (interleaved): the chunks form blocks of ILV chunks
// (the last one possibly shorter, nb chunks), each block covering 4*RPW*nb consecutive neurons, and
// chunk g of a block takes its neurons g, g + nb, g + 2 nb, ...  The low-indexed hot neurons of a
// hot-first layer then spread over the first block's chunks, while a chunk's Q rows stay within one
// block (a few MB) instead of spanning the whole matrix, which streamed measurably slower on MI355X.
// All the chunk's Q row loads are issued first, h (fp32, [nb][r], zero past r) is staged in LDS
// once per workgroup, then every lane forms its partial dot products and the wave sums them.  A
// neuron's logit does not depend on which chunk computes it.
// Neurons below n_hot are kept without a test (their Q rows are not read; their logits are
// unspecified).  Writes the logits when asked, and returns the chunk's kept-neuron bits in every
// thread.  Contains barriers: every thread of the workgroup calls it.
template <int ILV, int RPW>
__device__ __forceinline__ int chunk_neuron(int q, int NC, int k) {
  if constexpr (ILV == 0) {
    return q * 4 * RPW + k;
  } else {
    const int G = q / ILV, g = q - G * ILV;
    const int nb = NC - G * ILV < ILV ? NC - G * ILV : ILV;
    return G * ILV * 4 * RPW + g + nb * k;
  }
}

template <St PT, int NB, int RV, int RPW, int ILV = 0>
__device__ __forceinline__ uint32_t q_chunk(const void* __restrict__ Q, const float* __restrict__ c,
                                            const float* __restrict__ h, int r, int F, float thr, int nb,
                                            float* __restrict__ logits, int n_hot, int q, int NC = 0) {
  constexpr int EPL = Tr<PT>::EPL;
  constexpr int ESZ = Tr<PT>::ESZ;
  __shared__ uint32_t s_mask[kBlock / kWave];
  const int lane = wave_lane(), wv = wave_id();
  // h (all tokens, fp32, zero past r) goes through LDS once per workgroup: the four waves share it.
  // Its loads go out before the Q rows (loads return in issue order), so the staging does not wait
  // for the rows.
  constexpr int HR = RV * kWave * EPL;  // h elements per token covered by the lanes' slices
  constexpr int HPT = (NB * HR / 4 + kBlock - 1) / kBlock;  // float4 of h per thread
  __shared__ float4 s_h[NB * HR / 4];
  float4 hs[HPT];
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    const int k = threadIdx.x + u * kBlock;
    const int b = k / (HR / 4), e = (k % (HR / 4)) * 4;  // r % 8 == 0: whole float4s
    hs[u] = k < NB * HR / 4 && b < nb && e < r ? *reinterpret_cast<const float4*>(h + (size_t)b * r + e)
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  uint4 qv[RPW][RV];
#pragma unroll
  for (int k = 0; k < RPW; ++k)
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int i = chunk_neuron<ILV, RPW>(q, NC, wv * RPW + k), e = v * kWave * EPL + lane * EPL;
      qv[k][v] = q_ld16z(reinterpret_cast<const char*>(Q) + ((size_t)i * r + e) * ESZ, i < F && i >= n_hot && e < r);
    }
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    const int k = threadIdx.x + u * kBlock;
    if (k < NB * HR / 4) s_h[k] = hs[u];
  }
  __syncthreads();
  float hv[NB][RV][EPL];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int e = v * kWave * EPL + lane * EPL;
      const float4 a0 = s_h[(b * HR + e) / 4];
      hv[b][v][0] = a0.x; hv[b][v][1] = a0.y; hv[b][v][2] = a0.z; hv[b][v][3] = a0.w;
      if constexpr (EPL == 8) {
        const float4 a1 = s_h[(b * HR + e) / 4 + 1];
        hv[b][v][4] = a1.x; hv[b][v][5] = a1.y; hv[b][v][6] = a1.z; hv[b][v][7] = a1.w;
      }
    }
  uint32_t mask = 0;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int i = chunk_neuron<ILV, RPW>(q, NC, wv * RPW + k);
    const float ci = i < F ? c[i] : 0.f;
    bool on = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < RV; ++v) {
        if constexpr (PT == St::F16) {
          acc = dot8_f16_f32(qv[k][v], make_float4(hv[b][v][0], hv[b][v][1], hv[b][v][2], hv[b][v][3]),
                             make_float4(hv[b][v][4], hv[b][v][5], hv[b][v][6], hv[b][v][7]), acc);
        } else {
          acc = fmaf(__uint_as_float(qv[k][v].x), hv[b][v][0], acc);
          acc = fmaf(__uint_as_float(qv[k][v].y), hv[b][v][1], acc);
          acc = fmaf(__uint_as_float(qv[k][v].z), hv[b][v][2], acc);
          acc = fmaf(__uint_as_float(qv[k][v].w), hv[b][v][3], acc);
        }
      }
      const float l = wave_sum(acc) + ci;
      if (b < nb) {
        on |= l > thr;
        if (logits && lane == 0 && i < F) logits[(size_t)b * F + i] = l;
      }
    }
    if ((on || i < n_hot) && i < F) mask |= 1u << k;
  }
  if (lane == 0) s_mask[wv] = mask;
  __syncthreads();
  return s_mask[0] | (s_mask[1] << RPW) | (s_mask[2] << (2 * RPW)) | (s_mask[3] << (3 * RPW));
}

// The chunk's bits into the mask words.  Chunks of 16 neurons write the halves of the 32-bit words
// (little endian); an odd last chunk writes its whole word, so the unused upper half reads as zero.
template <int ROWS>
__device__ __forceinline__ void store_chunk_bits(uint32_t* masks, int q, int NQ, uint32_t bits) {
  static_assert(ROWS == 32 || ROWS == 16, "chunks of 32 or 16 neurons");
  if constexpr (ROWS == 32) {
    masks[q] = bits;
  } else if ((q & 1) == 0 && q == NQ - 1) {
    masks[q >> 1] = bits;
  } else {
    reinterpret_cast<uint16_t*>(masks)[q] = (uint16_t)bits;
  }
}

}  // namespace psffn

// Small-batch pipeline (B <= 4), four kernels per layer:
//
//   k_h     h = A x                       one wave per row of A, all of a row's loads in flight
//   k_q     l = Q h + c, threshold, and the ascending active list by decoupled look-back
//   k_up    a_k = act(W_up[idx[k]] . x (+ gate branch))   one wave per listed neuron
//   k_down  column tile x k-split partial sums of a_k * W_dT[idx[k]]
//   k_reduce_splits  y = b_down + the partials summed in split order (+ y when accumulating)
//
// Method ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur
// Research summary): Summary 2nd paragraph (a per-layer predictor guesses the firing neurons;
// neuron-level kernels compute those and skip the rest) and Interesting ideas I4 (work directly
// on whole weight rows and columns).
//
// Why kernel boundaries and not in-kernel waits: measured on MI355X, a dependency resolved inside
// a kernel costs a coherent memory round trip while every HBM queue is full (several µs), and a
// shared counter that ~1000 workgroups touch serialises at ~7 ns per access.  A kernel boundary
// costs ~1.5 µs.  The only in-kernel wait left is the look-back of k_q, where chunks finish
// staggered in dispatch order and a chunk usually finds its predecessor's prefix already
// published.
//
// Cross-workgroup words (look-back states, tile counters, partial sums) are read and written
// with relaxed device-scope atomics: on gfx950 those carry the sc1 bit, each access is coherent
// across the XCDs' separate L2 caches on its own, and polling them costs no cache maintenance.
// A writer waits for its data stores to complete (s_waitcnt) before bumping a counter; a reader
// loads data only after it has observed the counter.
#include "common.h"

namespace psffn {

constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_relaxed(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_relaxed(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this wave's outstanding memory operations (the published data) have completed
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0); }

// Value of a state word (epoch << 32 | value) once it carries this call's epoch.  Bounded: on
// timeout the error bit is set and 0 is returned.
__device__ __forceinline__ uint32_t wait_epoch(const unsigned long long* p, unsigned long long epoch, uint32_t* err) {
  unsigned long long w = ld_relaxed(p);
  uint32_t it = 0;
  while ((w >> 32) != epoch && it++ < kSpinLimit) {
    __builtin_amdgcn_s_sleep(1);
    w = ld_relaxed(p);
  }
  if ((w >> 32) != epoch) {
    atomicOr(err, 2u);
    return 0u;
  }
  return (uint32_t)w;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// rows per k-split of the down projection for a list of n >= 0 neurons, and the split count
// (>= 1; an empty list still has one, empty, split so that every column tile gets reduced)
__device__ __forceinline__ void ffn_split(int n, int& ks, int& S) {
  ks = (n + kSplitCap - 1) / kSplitCap;
  if (ks < 32) ks = 32;
  S = n > 0 ? (n + ks - 1) / ks : 1;
}

constexpr int kStageX = 65536;  // bytes of LDS for the activations of all tokens (B * d * elem)

// Copy n bytes of activations into LDS (16-byte pieces, all in flight at once), then barrier.
__device__ __forceinline__ void stage_x(const void* __restrict__ x, size_t n, uint4* s_x) {
  const uint4* src = reinterpret_cast<const uint4*>(x);
  const int n16 = (int)(n / 16);
  for (int k0 = threadIdx.x; k0 < n16; k0 += 8 * kBlock) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = k0 + u * kBlock < n16 ? src[k0 + u * kBlock] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u * kBlock < n16) s_x[k0 + u * kBlock] = v[u];
  }
  __syncthreads();
}

// =========================================================================================
// k_h: h[b][j] = A[j] . x_b.  One wave per row, up to 16 slices of 16 B in flight per lane.
// Block 0 also advances the call epoch that tags this call's look-back states.

template <St PT, int NB>
__global__ __launch_bounds__(kBlock) void k_h(const void* __restrict__ A, const void* __restrict__ x, int d, int r,
                                              int nb, float* __restrict__ h, uint32_t* __restrict__ hdr) {
  constexpr int EPL = Tr<PT>::EPL;
  constexpr int ESZ = Tr<PT>::ESZ;
  constexpr int UN = 16;
  extern __shared__ uint4 s_x[];  // B * d activations (dynamic size)
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr[kEpoch] = hdr[kEpoch] + 1u;
  const int lane = wave_lane();
  const int j = blockIdx.x * (kBlock / kWave) + wave_id();
  const char* arow = reinterpret_cast<const char*>(A) + (size_t)(j < r ? j : 0) * d * ESZ;
  // this wave's row loads go out first, then the workgroup stages x (all tokens) in LDS
  uint4 w[UN];
  int base = lane * EPL;
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const int e = base + u * kWave * EPL;
    w[u] = (j < r && e < d) ? ld16(arow + (size_t)e * ESZ) : make_uint4(0, 0, 0, 0);
  }
  stage_x(x, (size_t)nb * d * ESZ, s_x);
  if (j >= r) return;
  const char* xs = reinterpret_cast<const char*>(s_x);
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  for (;;) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int e = base + u * kWave * EPL;
      if (e < d) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < nb) acc[b] = dot16<PT>(w[u], xs + (size_t)b * d * ESZ, e, 1.f, acc[b]);
      }
    }
    base += UN * kWave * EPL;
    if (base >= d) break;
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int e = base + u * kWave * EPL;
      w[u] = e < d ? ld16(arow + (size_t)e * ESZ) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float s = wave_sum(acc[b]);
    if (lane == 0 && b < nb) h[(size_t)b * r + j] = s;
  }
}

// =========================================================================================
// k_q: chunk q = blockIdx.x covers neurons [q*4*RPW, (q+1)*4*RPW), RPW per wave.  All Q row
// loads are issued first; h (fp32, from the previous kernel) is read next; then logits, the
// union test over the batch, and the chunk's place in the ascending list.

template <St PT, int NB, int RV, int RPW, bool MASKS>
__global__ __launch_bounds__(kBlock) void k_q(const void* __restrict__ Q, const float* __restrict__ c,
                                              const float* __restrict__ h, int r, int F, float thr, int nb,
                                              uint32_t* __restrict__ hdr, unsigned long long* __restrict__ cstate,
                                              unsigned long long* __restrict__ gstate, int32_t* __restrict__ idx,
                                              int32_t* __restrict__ count, float* __restrict__ logits, int NQ,
                                              uint32_t* __restrict__ masks) {
  constexpr int EPL = Tr<PT>::EPL;
  constexpr int ESZ = Tr<PT>::ESZ;
  constexpr int ROWS = 4 * RPW;
  __shared__ uint32_t s_mask[kBlock / kWave];
  __shared__ int s_base;
  const int lane = wave_lane(), wv = wave_id();
  const int q = blockIdx.x;
  const int i0 = q * ROWS + wv * RPW;
  uint4 qv[RPW][RV];
#pragma unroll
  for (int k = 0; k < RPW; ++k)
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int i = i0 + k, e = v * kWave * EPL + lane * EPL;
      qv[k][v] = (i < F && e < r) ? ld16(reinterpret_cast<const char*>(Q) + ((size_t)i * r + e) * ESZ)
                                  : make_uint4(0, 0, 0, 0);
    }
  const unsigned long long epoch = hdr[kEpoch];
  float hv[NB][RV][EPL];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int e = v * kWave * EPL + lane * EPL;
#pragma unroll
      for (int k = 0; k < EPL; ++k) hv[b][v][k] = 0.f;
      if (b < nb && e < r) {
        const float* hp = h + (size_t)b * r + e;
        const float4 a0 = *reinterpret_cast<const float4*>(hp);
        hv[b][v][0] = a0.x; hv[b][v][1] = a0.y; hv[b][v][2] = a0.z; hv[b][v][3] = a0.w;
        if constexpr (EPL == 8) {
          const float4 a1 = *reinterpret_cast<const float4*>(hp + 4);
          hv[b][v][4] = a1.x; hv[b][v][5] = a1.y; hv[b][v][6] = a1.z; hv[b][v][7] = a1.w;
        }
      }
    }
  uint32_t mask = 0;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int i = i0 + k;
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
    if (on && i < F) mask |= 1u << k;
  }
  if (lane == 0) s_mask[wv] = mask;
  __syncthreads();
  if constexpr (MASKS) {
    // layer path: publish the chunk's active bits only; the up kernel orders them
    static_assert(4 * RPW == 32, "one 32-bit mask word per chunk");
    if (threadIdx.x == 0) masks[q] = s_mask[0] | (s_mask[1] << RPW) | (s_mask[2] << (2 * RPW)) | (s_mask[3] << (3 * RPW));
    return;
  }
  int cnt = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) cnt += __popc(s_mask[w]);
  // ---- place in the ascending list: a two-level scan.  Chunk q publishes its count; wave 0
  // reads the counts of the earlier chunks of its group of 64 (one load per lane); the last
  // chunk of a group publishes the group total; the chunk then reads the totals of the earlier
  // groups (one load per lane per 64 groups).  No dependency chain is longer than one group, so
  // chunks that all finish together do not walk back one window at a time.  Words are tagged
  // with the call epoch: a word from an earlier call counts as not yet published.
  if (wv == 0) {
    const unsigned long long tag = epoch << 32;
    if (lane == 0) st_relaxed(&cstate[q], tag | (uint32_t)cnt);
    const int g = q / kWave;
    int pre = 0;
    {
      const int jj = g * kWave + lane;
      uint32_t v = 0;
      if (jj < q) v = wait_epoch(&cstate[jj], epoch, &hdr[kErr]);
      pre = wave_sum_int((int)v);
    }
    if (q % kWave == kWave - 1 || q == NQ - 1) {
      if (lane == 0) st_relaxed(&gstate[g], tag | (uint32_t)(pre + cnt));
    }
    for (int g0 = 0; g0 < g; g0 += kWave) {
      const int gg = g0 + lane;
      uint32_t v = 0;
      if (gg < g) v = wait_epoch(&gstate[gg], epoch, &hdr[kErr]);
      pre += wave_sum_int((int)v);
    }
    if (lane == 0) s_base = pre;
  }
  __syncthreads();
  int wpre = 0;
  for (int w = 0; w < wv; ++w) wpre += __popc(s_mask[w]);
  const uint32_t m = s_mask[wv];
  if (lane < RPW && ((m >> lane) & 1u)) {
    const int at = s_base + wpre + __popc(m & ((1u << lane) - 1u));
    if (at < F) idx[at] = i0 + lane;
  }
  if (q == NQ - 1 && threadIdx.x == 0) *count = min(s_base + cnt, F);
}

// =========================================================================================
// FFN

template <St WT> struct DownTile;
template <> struct DownTile<St::F32> { static constexpr int CPL = 4; };
template <> struct DownTile<St::F16> { static constexpr int CPL = 8; };
template <> struct DownTile<St::I4> { static constexpr int CPL = 16; };

constexpr int kMaxScanChunks = 8192;  // chunks of 32 neurons the layer path can order (F <= 262144)

struct FfnArgs {
  const uint32_t* masks;  // layer path: per-chunk active bits from k_q
  int32_t* idx_out;       // layer path: the ascending list written by k_up
  int32_t* count_out;
  int nq;
  size_t xbytes;
  const void* w_up;
  const void* w_gate;
  const void* w_dT;
  const void* s_up;
  const void* s_gate;
  const void* s_dT;
  const float* b_up;
  const float* b_gate;
  const float* b_down;
  const void* x;
  const int32_t* idx;
  const int32_t* count;
  float* a;
  float* part;
  uint32_t* hdr;
  uint32_t* tile_done;
  float* y;
  int B, d, F, accumulate;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + expf(-g)); }

template <St WT>
__device__ __forceinline__ float group_scale(const void* s, int i, int d, int e) {
  if constexpr (WT == St::I4) {
    return h2f(reinterpret_cast<const uint16_t*>(s)[(size_t)i * (d / 128) + e / 128]);
  } else {
    return 1.f;
  }
}

__device__ __forceinline__ int list_len(const int32_t* count, int F) {
  const int n = *count;
  return n < 0 ? 0 : (n > F ? F : n);
}

// k_up: a[k][b] for every listed neuron k < count (grid-stride, one wave per neuron).  The row
// loads of the wave's first neuron go out before the workgroup stages x in LDS.
// SCAN mode of k_up: the chunk mask words are copied to LDS with coalesced loads (all in flight),
// then s_pre[q] = number of active neurons in chunks before q, s_pre[nq] = total.
__device__ void chunk_prefix(const uint32_t* __restrict__ masks, int nq, uint32_t* s_mask, int* s_pre, int* s_red) {
  for (int q0 = threadIdx.x; q0 < nq; q0 += 8 * kBlock) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = q0 + u * kBlock < nq ? masks[q0 + u * kBlock] : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u * kBlock < nq) s_mask[q0 + u * kBlock] = v[u];
  }
  __syncthreads();
  const int per = (nq + kBlock - 1) / kBlock;  // consecutive chunks per thread
  const int q0 = threadIdx.x * per;
  int tot = 0;
  for (int u = 0; u < per; ++u)
    if (q0 + u < nq) tot += __popc(s_mask[q0 + u]);
  // inclusive scan of the per-thread totals: within the wave, then across the 4 waves
  const int lane = wave_lane(), wv = wave_id();
  int inc = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == kWave - 1) s_red[wv] = inc;
  __syncthreads();
  int run = inc - tot;
  for (int w = 0; w < wv; ++w) run += s_red[w];
  for (int u = 0; u < per; ++u)
    if (q0 + u < nq) {
      s_pre[q0 + u] = run;
      run += __popc(s_mask[q0 + u]);
    }
  if (threadIdx.x == kBlock - 1) s_pre[nq] = run;
  __syncthreads();
}

// neuron at list position k, from the chunk prefix and mask words in LDS (binary search + bit select)
__device__ __forceinline__ int list_entry(const uint32_t* s_mask, const int* s_pre, int nq, int k) {
  int lo = 0, hi = nq - 1;  // last chunk with s_pre[q] <= k
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= k) lo = mid; else hi = mid - 1;
  }
  uint32_t m = s_mask[lo];
  for (int j = k - s_pre[lo]; j > 0; --j) m &= m - 1u;  // drop the j lowest set bits
  return lo * 32 + (int)__builtin_ctz(m);
}

template <St WT, psffn_act ACT, int NB, bool SCAN>
__global__ __launch_bounds__(kBlock) void k_up(FfnArgs g) {
  constexpr int EPL = Tr<WT>::EPL;
  constexpr int XSZ = WT == St::F32 ? 4 : 2;
  constexpr int UN = ACT == PSFFN_SWIGLU ? 8 : 16;
  extern __shared__ uint4 s_x[];  // B * d activations, then (SCAN) the chunk prefix
  __shared__ int s_red[kBlock / kWave];
  int n;
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s_x) + g.xbytes);
  int* s_pre = reinterpret_cast<int*>(s_mask + g.nq);
  if constexpr (SCAN) {
    chunk_prefix(g.masks, g.nq, s_mask, s_pre, s_red);
    n = min(s_pre[g.nq], g.F);
    if (blockIdx.x == 0 && threadIdx.x == 0) *g.count_out = n;
  } else {
    n = list_len(g.count, g.F);
  }
  if (blockIdx.x * (kBlock / kWave) >= n) return;  // no neuron for this workgroup
  const int lane = wave_lane();
  const size_t rb = row_bytes<WT>(g.d);
  const char* xs = reinterpret_cast<const char*>(s_x);
  bool staged = false;
  for (int k0 = blockIdx.x * (kBlock / kWave); k0 < n; k0 += gridDim.x * (kBlock / kWave)) {
    const int k = k0 + wave_id();
    int i = -1;
    if constexpr (SCAN) {
      if (k < n) {
        i = list_entry(s_mask, s_pre, g.nq, k);
        if (lane == 0) g.idx_out[k] = i;
      }
    } else {
      i = k < n ? g.idx[k] : -1;
    }
    const bool valid = (unsigned)i < (unsigned)g.F;
    const char* urow = reinterpret_cast<const char*>(g.w_up) + (size_t)(valid ? i : 0) * rb;
    const char* grow =
        ACT == PSFFN_SWIGLU ? reinterpret_cast<const char*>(g.w_gate) + (size_t)(valid ? i : 0) * rb : nullptr;
    float uacc[NB], gacc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) uacc[b] = gacc[b] = 0.f;
    uint4 wu[UN], wg[UN];
    int base = lane * EPL;
    // loads of a batch of UN slices; lanes past the end of the row load nothing
    auto load_batch = [&]() {
#pragma unroll
      for (int q = 0; q < UN; ++q) {
        const int e = base + q * kWave * EPL;
        const size_t off = WT == St::I4 ? (size_t)e / 2 : (size_t)e * Tr<WT>::ESZ;
        wu[q] = (valid && e < g.d) ? ld16(urow + off) : make_uint4(0, 0, 0, 0);
        if constexpr (ACT == PSFFN_SWIGLU) wg[q] = (valid && e < g.d) ? ld16(grow + off) : make_uint4(0, 0, 0, 0);
      }
    };
    load_batch();
    // every thread of the workgroup takes part in staging x (uniform: first neuron of the block)
    if (!staged) {
      stage_x(g.x, (size_t)g.B * g.d * XSZ, s_x);
      staged = true;
    }
    for (;;) {
#pragma unroll
      for (int q = 0; q < UN; ++q) {
        const int e = base + q * kWave * EPL;
        if (valid && e < g.d) {
          const float su = group_scale<WT>(g.s_up, i, g.d, e);
          float sg = 1.f;
          if constexpr (ACT == PSFFN_SWIGLU) sg = group_scale<WT>(g.s_gate, i, g.d, e);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (b < g.B) {
              const char* xr = xs + (size_t)b * g.d * XSZ;
              uacc[b] = dot16<WT>(wu[q], xr, e, su, uacc[b]);
              if constexpr (ACT == PSFFN_SWIGLU) gacc[b] = dot16<WT>(wg[q], xr, e, sg, gacc[b]);
            }
        }
      }
      base += UN * kWave * EPL;
      if (base >= g.d) break;
      load_batch();
    }
    const float bu = (valid && g.b_up) ? g.b_up[i] : 0.f;
    const float bg = (valid && g.b_gate) ? g.b_gate[i] : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float uu = wave_sum(uacc[b]) + bu;
      float av;
      if constexpr (ACT == PSFFN_SWIGLU) {
        av = silu_f(wave_sum(gacc[b]) + bg) * uu;
      } else {
        av = uu > 0.f ? uu : 0.f;
      }
      if (!valid) av = 0.f;
      if (lane == 0 && b < g.B && k < n) g.a[(size_t)k * g.B + b] = av;
    }
  }
}

// Issue the loads of PF rows k0, k0+4, ... of the list for this lane's columns: all PF indices
// first, then all PF weight slices, so a batch costs two memory round trips, not 2*PF.
template <St WT, int PF>
__device__ __forceinline__ void down_batch_load(const FfnArgs& g, int k0, int k_hi, int col0, bool live,
                                                uint4 (&wr)[PF], float (&sc)[PF], int (&rows)[PF]) {
#pragma unroll
  for (int p = 0; p < PF; ++p) rows[p] = k0 + 4 * p < k_hi ? g.idx[k0 + 4 * p] : -1;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    int i = rows[p];
    if ((unsigned)i >= (unsigned)g.F) i = -1;
    rows[p] = i;
    wr[p] = make_uint4(0, 0, 0, 0);
    sc[p] = 1.f;
    if (i >= 0 && live) {
      if constexpr (WT == St::F32) {
        wr[p] = ld16(reinterpret_cast<const float*>(g.w_dT) + (size_t)i * g.d + col0);
      } else if constexpr (WT == St::F16) {
        wr[p] = ld16(reinterpret_cast<const uint16_t*>(g.w_dT) + (size_t)i * g.d + col0);
      } else {
        uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(g.w_dT) + (size_t)i * (g.d / 2) +
                                                  col0 / 2);
        wr[p] = make_uint4(v.x, v.y, 0, 0);
        sc[p] = group_scale<WT>(g.s_dT, i, g.d, col0);
      }
    }
  }
}

constexpr int kActStage = 4096;  // floats of LDS for one split's activations (rows x batch)

// k_down: workgroup (tile, s) = column tile x k-split; its 4 waves take the split's rows round
// robin (PF rows in flight per wave) and are combined in wave order through LDS into the split's
// partial.  (A last-arriving split reducing the tile inside this kernel was measured slower: the
// coherent store, counter and load round trips cost ~8 us after the weights had streamed.)
template <St WT, int NB>
__global__ __launch_bounds__(kBlock) void k_down(FfnArgs g) {
  constexpr int CPL = DownTile<WT>::CPL;
  constexpr int TW = kWave * CPL;
  constexpr int PF = 8;
  __shared__ float s_acc[NB * TW];
  __shared__ float s_a[kActStage];
  const int n = list_len(g.count, g.F);
  int ks, S;
  ffn_split(n, ks, S);
  const int s = blockIdx.y, tile = blockIdx.x;
  if (s >= S) return;
  const int lane = wave_lane(), wv = wave_id();
  const int col0 = tile * TW + lane * CPL;
  const bool live = col0 < g.d;
  const int k_lo = s * ks;
  const int k_hi = min(n, k_lo + ks);
  uint4 wr[PF];
  float sc[PF];
  int rows[PF];
  down_batch_load<WT, PF>(g, k_lo + wv, k_hi, col0, live, wr, sc, rows);
  // the split's activations a[k_lo..k_hi) x B, 8 loads in flight per thread
  const int na = (k_hi - k_lo) * g.B;
  for (int q0 = threadIdx.x; q0 < na; q0 += 8 * kBlock) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = q0 + u * kBlock < na ? g.a[(size_t)k_lo * g.B + q0 + u * kBlock] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u * kBlock < na) s_a[q0 + u * kBlock] = v[u];
  }
  __syncthreads();
  float acc[NB][CPL];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[b][e] = 0.f;
  for (int k0 = k_lo + wv; k0 < k_hi; k0 += 4 * PF) {
    if (k0 != k_lo + wv) down_batch_load<WT, PF>(g, k0, k_hi, col0, live, wr, sc, rows);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int k = k0 + 4 * p;
      if (rows[p] < 0) continue;
      float w[CPL];
      if constexpr (WT == St::F32) {
        w[0] = __uint_as_float(wr[p].x); w[1] = __uint_as_float(wr[p].y);
        w[2] = __uint_as_float(wr[p].z); w[3] = __uint_as_float(wr[p].w);
      } else if constexpr (WT == St::F16) {
        w[0] = h2f(wr[p].x & 0xffff); w[1] = h2f(wr[p].x >> 16); w[2] = h2f(wr[p].y & 0xffff);
        w[3] = h2f(wr[p].y >> 16); w[4] = h2f(wr[p].z & 0xffff); w[5] = h2f(wr[p].z >> 16);
        w[6] = h2f(wr[p].w & 0xffff); w[7] = h2f(wr[p].w >> 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = i4_elem(wr[p].x, e) * sc[p];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[8 + e] = i4_elem(wr[p].y, e) * sc[p];
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < g.B) {
          const float ab = s_a[(k - k_lo) * g.B + b];
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[b][e] = fmaf(ab, w[e], acc[b][e]);
        }
    }
  }
  // combine the 4 waves in wave order through LDS; the partial goes out with plain stores (the
  // reduce kernel reads it after the kernel boundary)
  for (int step = 0; step < kBlock / kWave; ++step) {
    if (wv == step) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int at = b * TW + lane * CPL + e;
          const float v = step == 0 ? acc[b][e] : s_acc[at] + acc[b][e];
          if (step < kBlock / kWave - 1)
            s_acc[at] = v;
          else if (live && b < g.B)
            g.part[((size_t)s * g.B + b) * g.d + col0 + e] = v;
        }
    }
    if (step < kBlock / kWave - 1) __syncthreads();
  }
}

// k_reduce: y[b][j] = (accumulate ? y[b][j] : 0) + (b_down[j] + sum_{s < S} part[s][b][j]), the
// sum in split order.  One thread per output; all of its partial loads in flight at once.
__global__ __launch_bounds__(kBlock) void k_reduce_splits(FfnArgs g) {
  const int n = list_len(g.count, g.F);
  int ks, S;
  ffn_split(n, ks, S);
  const size_t t = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (size_t)g.B * g.d) return;
  const int b = (int)(t / g.d), col = (int)(t % g.d);
  float v = g.b_down ? g.b_down[col] : 0.f;
  for (int s0 = 0; s0 < S; s0 += 32) {
    float pv[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) pv[u] = s0 + u < S ? g.part[((size_t)(s0 + u) * g.B + b) * g.d + col] : 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u)
      if (s0 + u < S) v += pv[u];
  }
  g.y[t] = g.accumulate ? g.y[t] + v : v;
}

// =========================================================================================
// launchers

template <St PT, int NB, int RV>
static hipError_t predict_t(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx, int32_t* count,
                            float* logits, void* ws, hipStream_t s) {
  constexpr int RPW = 8;
  const StateLayout L = state_layout(P.F);
  char* w = static_cast<char*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(w);
  unsigned long long* cstate = reinterpret_cast<unsigned long long*>(w + L.chunk_state);
  unsigned long long* gstate = reinterpret_cast<unsigned long long*>(w + L.group_state);
  float* h = reinterpret_cast<float*>(w + L.scratch);
  const int NQ = (P.F + 4 * RPW - 1) / (4 * RPW);
  if ((size_t)B * P.d * Tr<PT>::ESZ > (size_t)kStageX) return hipErrorNotSupported;
  const size_t xbytes = round256((size_t)B * P.d * Tr<PT>::ESZ);
  k_h<PT, NB><<<(P.r + 3) / 4, kBlock, xbytes, s>>>(P.A, x, P.d, P.r, B, h, hdr);
  k_q<PT, NB, RV, RPW, false><<<NQ, kBlock, 0, s>>>(P.Q, P.c, h, P.r, P.F, thr, B, hdr, cstate, gstate, idx, count,
                                                    logits, NQ, nullptr);
  return hipGetLastError();
}

template <St PT, int NB>
static hipError_t predict_rv(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx, int32_t* count,
                             float* logits, void* ws, hipStream_t s) {
  const int per = kWave * Tr<PT>::EPL;  // elements of a row covered by one 16-byte slice per lane
  const int rv = (P.r + per - 1) / per;
  if (rv == 1) return predict_t<PT, NB, 1>(P, x, B, thr, idx, count, logits, ws, s);
  if (rv == 2) return predict_t<PT, NB, 2>(P, x, B, thr, idx, count, logits, ws, s);
  if (rv == 3) return predict_t<PT, NB, 3>(P, x, B, thr, idx, count, logits, ws, s);
  if (rv == 4) return predict_t<PT, NB, 4>(P, x, B, thr, idx, count, logits, ws, s);
  return hipErrorNotSupported;
}

template <St PT>
static hipError_t predict_nb(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx, int32_t* count,
                             float* logits, void* ws, hipStream_t s) {
  if (B == 1) return predict_rv<PT, 1>(P, x, B, thr, idx, count, logits, ws, s);
  if (B == 2) return predict_rv<PT, 2>(P, x, B, thr, idx, count, logits, ws, s);
  if (B <= 4) return predict_rv<PT, 4>(P, x, B, thr, idx, count, logits, ws, s);
  return hipErrorNotSupported;
}

hipError_t launch_predict_fused(St st, const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx,
                                int32_t* count, float* logits, void* ws, hipStream_t s) {
  if (st == St::F32) return predict_nb<St::F32>(P, x, B, thr, idx, count, logits, ws, s);
  if (st == St::F16) return predict_nb<St::F16>(P, x, B, thr, idx, count, logits, ws, s);
  return hipErrorNotSupported;
}

template <St WT>
static bool ffn_fits(const psffn_ffn& W, int B) {
  // the largest split (all F neurons listed) must fit the LDS activation stage, x must fit LDS
  int ks_max = (W.F + kSplitCap - 1) / kSplitCap;
  if (ks_max < 32) ks_max = 32;
  constexpr int TW = kWave * DownTile<WT>::CPL;
  return ks_max * B <= kActStage && (W.d + TW - 1) / TW <= kMaxTiles &&
         (size_t)B * W.d * (WT == St::F32 ? 4 : 2) <= (size_t)kStageX;
}

template <St WT>
static FfnArgs ffn_args(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count, float* y,
                        int accumulate, void* ws) {
  const StateLayout L = state_layout(W.F);
  char* w = static_cast<char*>(ws);
  FfnArgs g{};
  g.w_up = W.w_up;
  g.w_gate = W.w_gate;
  g.w_dT = W.w_dT;
  g.s_up = W.s_up;
  g.s_gate = W.s_gate;
  g.s_dT = W.s_dT;
  g.b_up = W.b_up;
  g.b_gate = W.b_gate;
  g.b_down = W.b_down;
  g.x = x;
  g.idx = idx;
  g.count = count;
  g.a = reinterpret_cast<float*>(w + L.scratch);
  g.part = reinterpret_cast<float*>(w + L.scratch + round256((size_t)W.F * B * 4));
  g.hdr = reinterpret_cast<uint32_t*>(w);
  g.tile_done = reinterpret_cast<uint32_t*>(w + L.tile_done);
  g.y = y;
  g.B = B;
  g.d = W.d;
  g.F = W.F;
  g.accumulate = accumulate;
  g.xbytes = round256((size_t)B * W.d * (WT == St::F32 ? 4 : 2));
  return g;
}

template <St WT, psffn_act ACT, int NB, bool SCAN>
static void ffn_launch(const FfnArgs& g, hipStream_t s) {
  constexpr int TW = kWave * DownTile<WT>::CPL;
  const int T = (g.d + TW - 1) / TW;
  int up_grid = (g.F + 3) / 4;
  if (up_grid > 1024) up_grid = 1024;
  const size_t lds = g.xbytes + (SCAN ? 4 * (size_t)(2 * g.nq + 1) : 0);
  k_up<WT, ACT, NB, SCAN><<<up_grid, kBlock, lds, s>>>(g);
  k_down<WT, NB><<<dim3(T, kSplitCap), kBlock, 0, s>>>(g);
  k_reduce_splits<<<(unsigned)(((size_t)g.B * g.d + kBlock - 1) / kBlock), kBlock, 0, s>>>(g);
}

template <St WT, psffn_act ACT, int NB>
static hipError_t ffn_t(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count, float* y,
                        int accumulate, void* ws, hipStream_t s) {
  if (!ffn_fits<WT>(W, B)) return hipErrorNotSupported;
  ffn_launch<WT, ACT, NB, false>(ffn_args<WT>(W, x, B, idx, count, y, accumulate, ws), s);
  return hipGetLastError();
}

template <St WT, psffn_act ACT>
static hipError_t ffn_nb(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count, float* y,
                         int accumulate, void* ws, hipStream_t s) {
  if (B == 1) return ffn_t<WT, ACT, 1>(W, x, B, idx, count, y, accumulate, ws, s);
  if (B == 2) return ffn_t<WT, ACT, 2>(W, x, B, idx, count, y, accumulate, ws, s);
  if (B <= 4) return ffn_t<WT, ACT, 4>(W, x, B, idx, count, y, accumulate, ws, s);
  return hipErrorNotSupported;
}

hipError_t launch_ffn_fused(St st, const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count,
                            float* y, int accumulate, void* ws, hipStream_t s) {
  if (W.act == PSFFN_RELU) {
    if (st == St::F32) return ffn_nb<St::F32, PSFFN_RELU>(W, x, B, idx, count, y, accumulate, ws, s);
    if (st == St::F16) return ffn_nb<St::F16, PSFFN_RELU>(W, x, B, idx, count, y, accumulate, ws, s);
    return ffn_nb<St::I4, PSFFN_RELU>(W, x, B, idx, count, y, accumulate, ws, s);
  }
  if (st == St::F32) return ffn_nb<St::F32, PSFFN_SWIGLU>(W, x, B, idx, count, y, accumulate, ws, s);
  if (st == St::F16) return ffn_nb<St::F16, PSFFN_SWIGLU>(W, x, B, idx, count, y, accumulate, ws, s);
  return ffn_nb<St::I4, PSFFN_SWIGLU>(W, x, B, idx, count, y, accumulate, ws, s);
}

// ---- one decode step of one layer: k_h, k_q (mask words only), k_up (orders the list from the
// masks, writes idx/count, computes the activations), k_down (partials + fixed-order reduce)

template <St PT, St WT, psffn_act ACT, int NB, int RV>
static hipError_t layer_t(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr, int32_t* idx,
                          int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s) {
  constexpr int RPW = 8;
  const int NQ = (P.F + 4 * RPW - 1) / (4 * RPW);
  // k_up's LDS: the activations plus 8 bytes per chunk must fit the default 64 KB allocation
  if (!ffn_fits<WT>(W, B) || NQ > kMaxScanChunks || (size_t)B * P.d * Tr<PT>::ESZ > (size_t)kStageX ||
      round256((size_t)B * W.d * (WT == St::F32 ? 4 : 2)) + 8 * (size_t)NQ + 4 > (size_t)65536)
    return hipErrorNotSupported;
  const StateLayout L = state_layout(P.F);
  char* w = static_cast<char*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(w);
  uint32_t* masks = reinterpret_cast<uint32_t*>(w + L.masks);
  float* h = reinterpret_cast<float*>(w + L.scratch);
  const size_t xbytes = round256((size_t)B * P.d * Tr<PT>::ESZ);
  k_h<PT, NB><<<(P.r + 3) / 4, kBlock, xbytes, s>>>(P.A, x, P.d, P.r, B, h, hdr);
  k_q<PT, NB, RV, RPW, true><<<NQ, kBlock, 0, s>>>(P.Q, P.c, h, P.r, P.F, thr, B, hdr, nullptr, nullptr, nullptr,
                                                   nullptr, logits, NQ, masks);
  FfnArgs g = ffn_args<WT>(W, x, B, idx, count, y, accumulate, ws);
  g.masks = masks;
  g.nq = NQ;
  g.idx_out = idx;
  g.count_out = count;
  ffn_launch<WT, ACT, NB, true>(g, s);
  return hipGetLastError();
}

template <St PT, St WT, psffn_act ACT, int NB>
static hipError_t layer_rv(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr, int32_t* idx,
                           int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s) {
  const int per = kWave * Tr<PT>::EPL;
  const int rv = (P.r + per - 1) / per;
  if (rv == 1) return layer_t<PT, WT, ACT, NB, 1>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (rv == 2) return layer_t<PT, WT, ACT, NB, 2>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (rv == 3) return layer_t<PT, WT, ACT, NB, 3>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (rv == 4) return layer_t<PT, WT, ACT, NB, 4>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  return hipErrorNotSupported;
}

template <St PT, St WT, psffn_act ACT>
static hipError_t layer_nb(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr, int32_t* idx,
                           int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s) {
  if (B == 1) return layer_rv<PT, WT, ACT, 1>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (B == 2) return layer_rv<PT, WT, ACT, 2>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (B <= 4) return layer_rv<PT, WT, ACT, 4>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  return hipErrorNotSupported;
}

template <St PT, St WT>
static hipError_t layer_act(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                            int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                            hipStream_t s) {
  if (W.act == PSFFN_RELU) return layer_nb<PT, WT, PSFFN_RELU>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  return layer_nb<PT, WT, PSFFN_SWIGLU>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
}

hipError_t launch_layer_fused(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                              int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                              hipStream_t s) {
  if (P.dt == PSFFN_F32 && W.dt == PSFFN_F32)
    return layer_act<St::F32, St::F32>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (P.dt == PSFFN_F16 && W.dt == PSFFN_F16)
    return layer_act<St::F16, St::F16>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  if (P.dt == PSFFN_F16 && W.dt == PSFFN_I4G128)
    return layer_act<St::F16, St::I4>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s);
  return hipErrorNotSupported;
}

}  // namespace psffn

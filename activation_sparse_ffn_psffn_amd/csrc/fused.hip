// Small-batch pipeline (B <= 4).  Layer call, four kernels:
//
//   k_h     h = A x                       one wave per row of A, all of a row's loads in flight
//   k_q     l = Q h + c, threshold; one bit per neuron (mask words, 16 neurons per workgroup)
//   k_ud    per split of the active list (ordered from the mask words in each workgroup):
//           a_k = act(W_up[idx[k]] . x (+ gate branch)), then the split's partial of
//           sum_k a_k W_dT[idx[k]]
//   k_reduce_ud  y = b_down + the split partials summed in split order (+ y when accumulating)
//
// The predictor call runs k_h, k_q and k_list (one workgroup: mask words -> ascending list);
// the FFN call runs k_ud from a given list, then k_reduce_ud.
//
// Method ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur
// Research summary): Summary 2nd paragraph (a per-layer predictor guesses the firing neurons;
// neuron-level kernels compute those and skip the rest) and Interesting ideas I4 (work directly
// on whole weight rows and columns).
//
// Why kernel boundaries and not in-kernel waits: measured on MI355X, back-to-back launches cost
// ~1-2 µs each, while a grid-wide barrier inside a persistent launch (one workgroup per CU, a
// device-scope counter polled with s_sleep) cost ~9 µs, more when the next phase's loads were
// already in flight.  So every cross-workgroup dependency is a kernel boundary; the up -> down
// dependency stays inside one workgroup of k_ud (its rows' activations never leave LDS).
//
// Loads are unconditional wherever the compiler would otherwise branch around them: a lane with
// nothing to load reads a 16-byte zero block instead.  A load behind a branch makes the compiler
// wait for every outstanding load at the join, which serialises independent row streams.
#include "chunk.h"
#include "common.h"

namespace psffn {

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// read through this block when a lane has nothing to load (keeps every load unconditional)
__device__ uint4 g_zero_ud[1] = {{0u, 0u, 0u, 0u}};  // never written

__device__ __forceinline__ uint4 ld16z(const void* p, bool ok) {
  return *reinterpret_cast<const uint4*>(ok ? p : static_cast<const void*>(g_zero_ud));
}
__device__ __forceinline__ uint2 ld8z(const void* p, bool ok) {
  return *reinterpret_cast<const uint2*>(ok ? p : static_cast<const void*>(g_zero_ud));
}
__device__ __forceinline__ uint32_t ld2z(const void* p, bool ok) {
  return (uint32_t)*reinterpret_cast<const uint16_t*>(ok ? p : static_cast<const void*>(g_zero_ud));
}
// Weight rows (A, the up, gate and down rows of the listed neurons) are read once per call: their
// loads are non-temporal, so that the stream does not push the reused lines (x, h, the mask words,
// the partials, the kernels' code) out of L2.  Each takes whole 128-byte lines in one instruction.
// Measured on MI355X (same machine, alternating): LLaMA2-13B-shaped SwiGLU layer at one token
// 65.3 -> 62.5 us and at four tokens 132.8 -> 129.8 us.
typedef unsigned int nt_u4v __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16z_nt(const void* p, bool ok) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                       reinterpret_cast<const nt_u4v*>(ok ? p : static_cast<const void*>(g_zero_ud))));
}
__device__ __forceinline__ uint2 ld8z_nt(const void* p, bool ok) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(
                                       reinterpret_cast<const nt_u2v*>(ok ? p : static_cast<const void*>(g_zero_ud))));
}


constexpr int kStageX = 65536;  // bytes of LDS for the activations of all tokens (B * d * elem)

// Copy n bytes of activations into LDS (16-byte pieces, all in flight at once), then barrier.
// NT = threads of the workgroup.
template <int NT>
__device__ __forceinline__ void stage_x(const void* __restrict__ x, size_t n, uint4* s_x) {
  const uint4* src = reinterpret_cast<const uint4*>(x);
  const int n16 = (int)(n / 16);
  for (int k0 = threadIdx.x; k0 < n16; k0 += 8 * NT) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = k0 + u * NT < n16 ? src[k0 + u * NT] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u * NT < n16) s_x[k0 + u * NT] = v[u];
  }
  __syncthreads();
}

// =========================================================================================
// k_h: h[b][j] = A[j] . x_b.  One wave per row, up to 16 slices of 16 B in flight per lane.
// (Two-wave workgroups, twice as many, measured 0.4 µs slower on a 1024 x 7168 fp16 A.)
constexpr int kHThreads = 256;

// LNK > 0 (fp16 predictor, stack step): x is the fp32 residual [nb][d]; every workgroup normalises
// it into LDS with ln_row_f16<LNK> (the LayerNorm kernel's arithmetic), and workgroup 0 also
// stores the fp16 rows to hout for the FFN kernel.
template <St PT, int NB, int LNK>
__global__ __launch_bounds__(kHThreads) void k_h(const void* __restrict__ A, const void* __restrict__ x, int d, int r,
                                              int nb, float* __restrict__ h, float eps, _Float16* __restrict__ hout,
                                              uint32_t* __restrict__ zero = nullptr, int nzero = 0,
                                              uint32_t* __restrict__ zero2 = nullptr, int nzero2 = 0) {
  constexpr int EPL = Tr<PT>::EPL;
  constexpr int ESZ = Tr<PT>::ESZ;
  constexpr int UN = 16;
  extern __shared__ uint4 s_x[];  // B * d activations (dynamic size)
  const int lane = wave_lane();
  const int j = blockIdx.x * (kHThreads / kWave) + wave_id();
  for (int k = blockIdx.x * kHThreads + threadIdx.x; k < nzero; k += gridDim.x * kHThreads) zero[k] = 0u;
  for (int k = blockIdx.x * kHThreads + threadIdx.x; k < nzero2; k += gridDim.x * kHThreads) zero2[k] = 0u;
  const char* arow = reinterpret_cast<const char*>(A) + (size_t)(j < r ? j : 0) * d * ESZ;
  // one token with the LayerNorm: the residual row's loads go out first, so that the LayerNorm's
  // reductions run while this wave's row of A is still in flight (loads return in issue order)
  static_assert(LNK == 0 || kHThreads == kBlock, "ln_row_* take kBlock threads");
  float4 xln[(LNK > 0 && NB == 1) ? LNK : 1];
  if constexpr (LNK > 0 && NB == 1) ln_row_load<LNK>(reinterpret_cast<const float*>(x), d, xln);
  // without the LayerNorm, x (all tokens) likewise goes out first when it is one round of 8 pieces
  // of 16 bytes per thread
  const int nx16 = (int)((size_t)nb * d * ESZ / 16);
  const bool x1r = LNK == 0 && nx16 <= 8 * kHThreads;
  uint4 xr8[LNK == 0 ? 8 : 1];
  if constexpr (LNK == 0) {
    if (x1r) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = threadIdx.x + u * kHThreads;
        xr8[u] = k < nx16 ? reinterpret_cast<const uint4*>(x)[k] : make_uint4(0, 0, 0, 0);
      }
    }
  }
  // this wave's row loads, then the workgroup stages x (all tokens) in LDS
  uint4 w[UN];
  int base = lane * EPL;
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const int e = base + u * kWave * EPL;
    w[u] = ld16z_nt(arow + (size_t)e * ESZ, j < r && e < d);
  }
  if constexpr (LNK > 0) {
    static_assert(PT == St::F16, "the LayerNorm output is fp16");
    __shared__ float s_red[kHThreads / kWave];
    if constexpr (NB == 1) {
      ln_row_finish<LNK>(xln, d, eps, s_red, reinterpret_cast<uint2*>(s_x));
    } else {
      for (int b = 0; b < nb; ++b)
        ln_row_f16<LNK>(reinterpret_cast<const float*>(x) + (size_t)b * d, d, eps, s_red,
                        reinterpret_cast<uint2*>(s_x) + (size_t)b * d / 4);
    }
    __syncthreads();
    if (blockIdx.x == 0) {
      const int n16 = nb * d / 8;  // d % 8 == 0
      for (int k = threadIdx.x; k < n16; k += kHThreads) reinterpret_cast<uint4*>(hout)[k] = s_x[k];
    }
  } else if (x1r) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = threadIdx.x + u * kHThreads;
      if (k < nx16) s_x[k] = xr8[u];
    }
    __syncthreads();
  } else {
    stage_x<kHThreads>(x, (size_t)nb * d * ESZ, s_x);
  }
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
      w[u] = ld16z_nt(arow + (size_t)e * ESZ, e < d);
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
// union test over the batch, and the chunk's mask bits.  Neurons below n_hot (the hot prefix of a
// hot-first layer) are kept without a test: their Q rows are not read, their bits are set, and
// their logits are left unspecified.

template <St PT, int NB, int RV, int RPW>
__global__ __launch_bounds__(kBlock) void k_q(const void* __restrict__ Q, const float* __restrict__ c,
                                              const float* __restrict__ h, int r, int F, float thr, int nb,
                                              float* __restrict__ logits, int NQ, uint32_t* __restrict__ masks,
                                              int n_hot) {
  constexpr int ROWS = 4 * RPW;
  const int q = blockIdx.x;
  if ((q + 1) * ROWS <= n_hot) {  // the whole chunk is hot (and below F)
    if (threadIdx.x == 0) store_chunk_bits<ROWS>(masks, q, NQ, ROWS == 32 ? 0xffffffffu : 0xffffu);
    return;
  }
  const uint32_t bits = q_chunk<PT, NB, RV, RPW>(Q, c, h, r, F, thr, nb, logits, n_hot, q);
  if (threadIdx.x == 0) store_chunk_bits<ROWS>(masks, q, NQ, bits);
}

// =========================================================================================
// k_list: one workgroup turns the mask words into the ascending list of active neurons and its
// length (the standalone predictor call; the layer call orders the list inside k_ud).  Thread t
// owns the consecutive words [t per, t per + per): a block scan of their popcounts gives its first
// list position, then it writes the ids of its words in order.

constexpr int kListThreads = 1024;

__global__ __launch_bounds__(kListThreads) void k_list(const uint32_t* __restrict__ masks, int nq, int F,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  extern __shared__ uint32_t s_m[];  // nq mask words
  __shared__ int s_red[kListThreads / kWave];
  for (int q = threadIdx.x; q < nq; q += kListThreads) s_m[q] = masks[q];
  __syncthreads();
  const int per = (nq + kListThreads - 1) / kListThreads;
  const int q0 = threadIdx.x * per;
  int tot = 0;
  for (int u = 0; u < per; ++u)
    if (q0 + u < nq) tot += __popc(s_m[q0 + u]);
  const int lane = wave_lane(), wv = wave_id();
  int inc = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == kWave - 1) s_red[wv] = inc;
  __syncthreads();
  int at = inc - tot, n = 0;
#pragma unroll
  for (int w = 0; w < kListThreads / kWave; ++w) {
    if (w < wv) at += s_red[w];
    n += s_red[w];
  }
  if (threadIdx.x == 0) *count = n < F ? n : F;
  for (int u = 0; u < per; ++u) {
    const int q = q0 + u;
    if (q >= nq) break;
    uint32_t m = s_m[q];
    while (m != 0u) {
      const int i = q * 32 + (int)__builtin_ctz(m);
      m &= m - 1u;
      if (at < F) idx[at] = i;
      ++at;
    }
  }
}

// =========================================================================================
// FFN


constexpr int kMaxScanChunks = 8192;  // chunks of 32 neurons the layer path can order (F <= 262144)

struct FfnArgs {
  const uint32_t* masks;  // layer path: per-chunk active bits from k_q
  int32_t* idx_out;       // layer path: the ascending list written by k_ud
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
  float* y;
  int B, d, F, accumulate;
  int n_hot;  // layer path: neurons [0, n_hot) are listed whatever the mask words say
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

// The layer call orders the list from the predictor's mask words (bit b of word q: neuron 32 q + b
// is active).  Thread t owns the consecutive words [t per, t per + per); a block scan of the
// per-thread popcounts gives every thread its first list position and the total, and each thread
// then emits the neuron ids of its words that fall in the workgroup's split, in ascending order.
// s_red holds the 4 wave totals.  Returns the list length (clamped to F).
__device__ __forceinline__ int scan_total(const uint32_t* s_mask, int nq, int F, int* s_red, int& first) {
  const int per = (nq + kBlock - 1) / kBlock;
  const int q0 = threadIdx.x * per;
  int tot = 0;
  for (int u = 0; u < per; ++u)
    if (q0 + u < nq) tot += __popc(s_mask[q0 + u]);
  const int lane = wave_lane(), wv = wave_id();
  int inc = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == kWave - 1) s_red[wv] = inc;
  __syncthreads();
  int run = inc - tot, n = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    if (w < wv) run += s_red[w];
    n += s_red[w];
  }
  first = run;
  return n < F ? n : F;
}

// ids of list positions [k_lo, k_hi) -> s_i[k - k_lo].  Each thread lists its words that
// intersect the range (word index and first position, packed as pos << 13 | q: q < 8192,
// pos <= 2^18) in s_wl; then lane j of a wave tests bit j of a listed word, so no thread walks
// bits one at a time.  *s_wn must be zero on entry; both passes end with a barrier.
__device__ __forceinline__ void scan_emit(const uint32_t* s_mask, int nq, int F, int first, int k_lo, int k_hi,
                                          int* s_i, uint32_t* s_wl, int* s_wn) {
  const int per = (nq + kBlock - 1) / kBlock;
  const int q0 = threadIdx.x * per;
  int pos = first;
  for (int u = 0; u < per; ++u) {
    const int q = q0 + u;
    const int c = q < nq ? __popc(s_mask[q]) : 0;
    if (c > 0 && pos < k_hi && pos + c > k_lo) s_wl[atomicAdd(s_wn, 1)] = ((uint32_t)pos << 13) | (uint32_t)q;
    pos += c;
  }
  __syncthreads();
  const int nw = *s_wn;
  const int lane = wave_lane();
  for (int j = wave_id(); j < nw; j += kBlock / kWave) {
    const uint32_t e = s_wl[j];
    const int q = (int)(e & 8191u), p0 = (int)(e >> 13);
    const uint32_t m = s_mask[q];
    if (lane < 32 && ((m >> lane) & 1u)) {
      const int at = p0 + __popc(m & ((1u << lane) - 1u));
      const int i = q * 32 + lane;
      if (at >= k_lo && at < k_hi) s_i[at - k_lo] = i < F ? i : -1;
    }
  }
  __syncthreads();
}

// =========================================================================================
// Fused up and down projection (one kernel instead of three): split s owns list positions
// [s ks, s ks + ks).  Its waves compute the activations of those rows (x in LDS), keep them in
// LDS, and the workgroup then streams the same rows of W_dT into a partial output
// part[s][b][col].  The up -> down dependency never leaves the workgroup; k_reduce_ud sums the S
// partials in split order.  The split depends on the list length only, so the summation order
// (and y) is a fixed function of (idx, count, shapes).
//
// Dense weights: one wave per up row (the whole row in flight), each thread owns 16-byte column
// slices of W_dT.  4-bit weights (rows of d/2 bytes, several per split): 32 lanes per up row, so
// a wave has 2 rows in flight, with the group scales requested beside the weights; in the down
// projection each thread owns 16-column units and decodes two rows at a time into fp16 pairs that
// feed fp32 dot2 products with (hi, lo) fp16 halves of activation x scale.

constexpr int kUDMaxRows = 1024;  // max rows of one split (F <= kUDSplitCap * kUDMaxRows)

// splits: enough to spread the rows over the CUs, few enough that the partials (S x B x d fp32,
// written then summed) stay near a quarter of the weight bytes the rows stream (half for 4-bit
// rows, whose decode is arithmetic-bound and wants the work spread over more CUs)
template <St WT>
__device__ __forceinline__ void udsplit(int n, int B, int d, int stream_bytes_per_row, int& ks, int& S) {
  constexpr int kDiv = WT == St::I4 ? 8 : 16;
  long long want = (long long)n * stream_bytes_per_row / ((long long)B * d * kDiv);
  if (want > kUDSplitCap) want = kUDSplitCap;
  if (want < 1) want = 1;
  ks = (int)((n + want - 1) / want);
  if (ks < 1) ks = 1;
  S = n > 0 ? (n + ks - 1) / ks : 1;
}

template <St WT>
__host__ __device__ inline int ud_stream_bytes(int d, psffn_act act) {
  const int rb = WT == St::F32 ? 4 * d : (WT == St::F16 ? 2 * d : d / 2 + 2 * (d / 128));
  return (act == PSFFN_SWIGLU ? 3 : 2) * rb;
}

// 4-bit decode with the sign bits pre-flipped (w ^ 0x88888888): the pair of nibbles at bits
// [s, s+4) and [16+s, 20+s) as fp16 (1024 + q + 8) - 1032 = q, exactly
__device__ __forceinline__ half2_t i4p(uint32_t wf, int s) {
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  return __builtin_bit_cast(half2_t, ((wf >> s) & 0x000F000Fu) | 0x64006400u) - off;
}

// sum of 32 products: one 16-byte slice of 4-bit weights x 32 fp16 activations stored pre-paired
// ((x0,x4),(x1,x5),(x2,x6),(x3,x7) per 8)
__device__ __forceinline__ float dot32_i4(uint4 w, const uint4* __restrict__ px) {
  const uint32_t ww[4] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u, w.z ^ 0x88888888u, w.w ^ 0x88888888u};
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4 p = px[k];
    acc = __builtin_amdgcn_fdot2(i4p(ww[k], 0), __builtin_bit_cast(half2_t, p.x), acc, false);
    acc = __builtin_amdgcn_fdot2(i4p(ww[k], 4), __builtin_bit_cast(half2_t, p.y), acc, false);
    acc = __builtin_amdgcn_fdot2(i4p(ww[k], 8), __builtin_bit_cast(half2_t, p.z), acc, false);
    acc = __builtin_amdgcn_fdot2(i4p(ww[k], 12), __builtin_bit_cast(half2_t, p.w), acc, false);
  }
  return acc;
}

__device__ __forceinline__ float sum32(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// fp32 -> (hi, lo) fp16 with hi + lo = v to ~22 bits
__device__ __forceinline__ void split_hl16(float v, _Float16& hi, _Float16& lo) {
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

template <St WT, psffn_act ACT, int NB, bool SCAN>
__global__ __launch_bounds__(kBlock) void k_ud(FfnArgs g) {
  constexpr int EPL = Tr<WT>::EPL;
  constexpr int XSZ = WT == St::F32 ? 4 : 2;
  constexpr int UN = ACT == PSFFN_SWIGLU ? 12 : 16;  // dense up: 16-byte slices per lane per pass
  extern __shared__ uint4 s_x[];  // x (B * d), then (SCAN) the mask words, then the split's rows
  __shared__ int s_red[kBlock / kWave];
  __shared__ int s_wn;
  char* dyn = reinterpret_cast<char*>(s_x);
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(dyn + g.xbytes);
  const size_t rows_off = g.xbytes + (SCAN ? round256(4 * (size_t)(2 * g.nq + 1)) : 0);
  float* s_a = reinterpret_cast<float*>(dyn + rows_off);                 // [kUDMaxRows][NB]
  int* s_i = reinterpret_cast<int*>(dyn + rows_off + 4 * (size_t)kUDMaxRows * NB);  // [kUDMaxRows]
  const int lane = wave_lane(), wv = wave_id();
  // ---- x (4-bit weights: paired for the dot2 decode) and the mask words go to LDS together
  {
    const int n16 = (int)((size_t)g.B * g.d * XSZ / 16);
    const uint4* src = reinterpret_cast<const uint4*>(g.x);
    if (threadIdx.x == 0) s_wn = 0;
    constexpr int MW = 8;
    uint32_t mv[MW];
    if constexpr (SCAN) {
#pragma unroll
      for (int u = 0; u < MW; ++u) {
        const int q = threadIdx.x + u * kBlock;
        mv[u] = q < g.nq ? g.masks[q] : 0u;
      }
    }
    for (int k0 = threadIdx.x; k0 < n16; k0 += 8 * kBlock) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = k0 + u * kBlock < n16 ? src[k0 + u * kBlock] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u * kBlock < n16) s_x[k0 + u * kBlock] = WT == St::I4 ? pair_x8(v[u]) : v[u];
    }
    if constexpr (SCAN) {
#pragma unroll
      for (int u = 0; u < MW; ++u) {
        const int q = threadIdx.x + u * kBlock;
        if (q < g.nq) s_mask[q] = mv[u];
      }
      for (int q = threadIdx.x + MW * kBlock; q < g.nq; q += kBlock) s_mask[q] = g.masks[q];
      // the hot prefix's bits (n_hot <= F: no bit past F is set)
      const int nwh = (g.n_hot + 31) / 32;
      for (int q = threadIdx.x; q < nwh; q += kBlock) {
        const int nh = g.n_hot - 32 * q;
        s_mask[q] |= nh >= 32 ? 0xffffffffu : (1u << nh) - 1u;
      }
    }
    __syncthreads();
  }
  // ---- the list length, this workgroup's split and its neuron ids
  int n, first = 0;
  if constexpr (SCAN) {
    n = scan_total(s_mask, g.nq, g.F, s_red, first);
  } else {
    n = list_len(g.count, g.F);
  }
  int ks, S;
  udsplit<WT>(n, g.B, g.d, ud_stream_bytes<WT>(g.d, ACT), ks, S);
  const int s = blockIdx.x;
  if (s >= S) return;
  const int k_lo = s * ks, k_hi = min(n, k_lo + ks);
  const int nr = k_hi > k_lo ? min(k_hi - k_lo, kUDMaxRows) : 0;
  if constexpr (SCAN) {
    // (s_a holds the word list until the up projection writes it: kUDMaxRows entries)
    scan_emit(s_mask, g.nq, g.F, first, k_lo, k_lo + nr, s_i, reinterpret_cast<uint32_t*>(s_a), &s_wn);
  } else {
    for (int kr = threadIdx.x; kr < nr; kr += kBlock) {
      const int i = g.idx[k_lo + kr];
      s_i[kr] = (unsigned)i < (unsigned)g.F ? i : -1;
    }
    __syncthreads();
  }
  const size_t rb = row_bytes<WT>(g.d);
  const char* xs = reinterpret_cast<const char*>(s_x);
  // the layer call's list and count are stored last: nothing in the kernel waits for them
  auto store_list = [&]() {
    if constexpr (SCAN) {
      for (int kr = threadIdx.x; kr < nr; kr += kBlock) {
        const int i = s_i[kr];
        g.idx_out[k_lo + kr] = i >= 0 ? i : 0;
      }
      if (s == 0 && threadIdx.x == 0) *g.count_out = n;
    }
  };
  if constexpr (WT == St::I4) {
    // ================= 4-bit weights
    const int ng = g.d / 128;
    const size_t srow = (size_t)ng * 2;  // bytes of one row's scales
    // ---- down: thread t owns 16-column units t + j kBlock (j < UJ) per pass; RBD rows per batch
    constexpr int UJ = NB == 1 ? 3 : 1;
    constexpr int RBD = 8;
    const int nu = g.d / 16;
    const char* wd = reinterpret_cast<const char*>(g.w_dT);
    const char* sd = reinterpret_cast<const char*>(g.s_dT);
    uint2 dw[RBD][UJ];
    uint32_t dsc[RBD][UJ];
    auto load_down = [&](int j0, int r0) {
#pragma unroll
      for (int r = 0; r < RBD; ++r) {
        const int i = r0 + r < nr ? s_i[r0 + r] : -1;
#pragma unroll
        for (int j = 0; j < UJ; ++j) {
          const int un = j0 + (int)threadIdx.x + j * kBlock;
          const bool ok = i >= 0 && un < nu;
          dw[r][j] = ld8z_nt(wd + (size_t)(ok ? i : 0) * rb + (size_t)un * 8, ok);
          dsc[r][j] = ld2z(sd + (size_t)(ok ? i : 0) * srow + (size_t)(un / 8) * 2, ok);
        }
      }
    };
    // ---- up: 32 lanes per row, 2 rows per wave, UQ 16-byte slices per lane per pass
    constexpr int UQ = 12;
    const int li = lane & 31, lg = lane >> 5;
    const int step = UQ * 32 * 32;
    const char* su_base = reinterpret_cast<const char*>(g.s_up);
    const char* sg_base = reinterpret_cast<const char*>(g.s_gate);
    uint4 wu[UQ], wg[UQ];
    uint32_t su[UQ], sg[UQ];
    float uacc[NB], gacc[NB];
    int i = -1;
    size_t ro = 0, so = 0;
    auto row_begin = [&](int k0) {
      const int kr = k0 + wv * 2 + lg;
      i = kr < nr ? s_i[kr] : -1;
      ro = (size_t)(i >= 0 ? i : 0) * rb;
      so = (size_t)(i >= 0 ? i : 0) * srow;
#pragma unroll
      for (int b = 0; b < NB; ++b) uacc[b] = gacc[b] = 0.f;
    };
    auto up_load = [&](int e0) {
#pragma unroll
      for (int q = 0; q < UQ; ++q) {
        const int e = e0 + (q * 32 + li) * 32;
        const bool ok = i >= 0 && e < g.d;
        wu[q] = ld16z_nt(reinterpret_cast<const char*>(g.w_up) + ro + e / 2, ok);
        su[q] = ld2z(su_base + so + (size_t)(e / 128) * 2, ok);
        if constexpr (ACT == PSFFN_SWIGLU) {
          wg[q] = ld16z_nt(reinterpret_cast<const char*>(g.w_gate) + ro + e / 2, ok);
          sg[q] = ld2z(sg_base + so + (size_t)(e / 128) * 2, ok);
        }
      }
    };
    auto up_acc = [&](int e0) {
#pragma unroll
      for (int q = 0; q < UQ; ++q) {
        const int e = e0 + (q * 32 + li) * 32;
        const int ec = e < g.d ? e : 0;  // (the weights and scales past d are zero)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < g.B) {
            const uint4* px = reinterpret_cast<const uint4*>(xs + ((size_t)b * g.d + ec) * 2);
            uacc[b] = fmaf(h2f(su[q]), dot32_i4(wu[q], px), uacc[b]);
            if constexpr (ACT == PSFFN_SWIGLU) gacc[b] = fmaf(h2f(sg[q]), dot32_i4(wg[q], px), gacc[b]);
          }
      }
    };
    auto row_end = [&](int k0) {
      const int kr = k0 + wv * 2 + lg;
      const bool valid = i >= 0;
      const float bu = (valid && g.b_up) ? g.b_up[i] : 0.f;
      const float bg = (valid && g.b_gate) ? g.b_gate[i] : 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float uu = sum32(uacc[b]) + bu;
        float av;
        if constexpr (ACT == PSFFN_SWIGLU) {
          av = silu_f(sum32(gacc[b]) + bg) * uu;
        } else {
          av = uu > 0.f ? uu : 0.f;
        }
        if (!valid || b >= g.B) av = 0.f;
        if (li == 0 && kr < nr) s_a[kr * NB + b] = av;
      }
    };
    // the first rows' first pass goes out before the first down batch, which then streams while
    // the up rows are reduced
    row_begin(0);
    up_load(0);
    load_down(0, 0);
    up_acc(0);
    for (int e0 = step; e0 < g.d; e0 += step) {
      up_load(e0);
      up_acc(e0);
    }
    row_end(0);
    for (int k0 = 2 * (kBlock / kWave); k0 < nr; k0 += 2 * (kBlock / kWave)) {
      row_begin(k0);
      for (int e0 = 0; e0 < g.d; e0 += step) {
        up_load(e0);
        up_acc(e0);
      }
      row_end(k0);
    }
    __syncthreads();
    // ---- down: two rows at a time, y[c] += (q_r, q_r') . (hi, hi') + (q_r, q_r') . (lo, lo')
    for (int j0 = 0; j0 < nu; j0 += UJ * kBlock) {
      if (j0 > 0) load_down(j0, 0);
      float acc[UJ][NB][16];
#pragma unroll
      for (int j = 0; j < UJ; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int c = 0; c < 16; ++c) acc[j][b][c] = 0.f;
      for (int r0 = 0; r0 < nr; r0 += RBD) {
        uint2 w[RBD][UJ];
        uint32_t sc[RBD][UJ];
#pragma unroll
        for (int r = 0; r < RBD; ++r)
#pragma unroll
          for (int j = 0; j < UJ; ++j) {
            w[r][j] = dw[r][j];
            sc[r][j] = dsc[r][j];
          }
        if (r0 + RBD < nr) load_down(j0, r0 + RBD);  // the next batch, if there is one
#pragma unroll
        for (int p = 0; p < RBD / 2; ++p) {
          const int r = r0 + 2 * p;
          if (r >= nr) continue;  // (no break: the loop must unroll, w[] stays in registers)
          float a0[NB], a1[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            a0[b] = s_a[r * NB + b];
            a1[b] = r + 1 < nr ? s_a[(r + 1) * NB + b] : 0.f;
          }
#pragma unroll
          for (int j = 0; j < UJ; ++j) {
            half2_t hp[NB], lp[NB];
            const float s0 = h2f(sc[2 * p][j]), s1 = h2f(sc[2 * p + 1][j]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              _Float16 h0, l0, h1, l1;
              split_hl16(a0[b] * s0, h0, l0);
              split_hl16(a1[b] * s1, h1, l1);
              hp[b] = half2_t{h0, h1};
              lp[b] = half2_t{l0, l1};
            }
            const uint32_t x0[2] = {w[2 * p][j].x ^ 0x88888888u, w[2 * p][j].y ^ 0x88888888u};
            const uint32_t x1[2] = {w[2 * p + 1][j].x ^ 0x88888888u, w[2 * p + 1][j].y ^ 0x88888888u};
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                // byte jj of both rows: columns 8h + 2jj (low nibbles) and 8h + 2jj + 1 (high)
                const uint32_t t = __builtin_amdgcn_perm(x1[h], x0[h], 0x0C000C00u | (uint32_t)jj | ((4u + jj) << 16));
                const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
                const half2_t vlo = __builtin_bit_cast(half2_t, (t & 0x000F000Fu) | 0x64006400u) - off;
                const half2_t vhi = __builtin_bit_cast(half2_t, ((t >> 4) & 0x000F000Fu) | 0x64006400u) - off;
                const int c = 8 * h + 2 * jj;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                  acc[j][b][c] = __builtin_amdgcn_fdot2(vlo, hp[b], acc[j][b][c], false);
                  acc[j][b][c] = __builtin_amdgcn_fdot2(vlo, lp[b], acc[j][b][c], false);
                  acc[j][b][c + 1] = __builtin_amdgcn_fdot2(vhi, hp[b], acc[j][b][c + 1], false);
                  acc[j][b][c + 1] = __builtin_amdgcn_fdot2(vhi, lp[b], acc[j][b][c + 1], false);
                }
              }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < UJ; ++j) {
        const int un = j0 + (int)threadIdx.x + j * kBlock;
        if (un >= nu) continue;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b >= g.B) continue;
          float* dst = g.part + ((size_t)s * g.B + b) * g.d + (size_t)un * 16;
#pragma unroll
          for (int c = 0; c < 16; c += 4)
            *reinterpret_cast<float4*>(dst + c) =
                make_float4(acc[j][b][c], acc[j][b][c + 1], acc[j][b][c + 2], acc[j][b][c + 3]);
        }
      }
    }
    store_list();
    return;
  } else {
    // ================= dense weights
    constexpr int CPL = WT == St::F32 ? 4 : 8;  // columns per 16-byte slice
    constexpr int UG = 32 / CPL;                // slices per thread per pass
    constexpr int RB = 16 / UG;                 // rows per batch
    const int nsl = g.d / CPL;                  // d % 8 == 0: whole slices
    const char* wd = reinterpret_cast<const char*>(g.w_dT);
    uint4 dw[RB][UG];
    auto load_down = [&](int j0, int r0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int i = r0 + r < nr ? s_i[r0 + r] : -1;
#pragma unroll
        for (int u = 0; u < UG; ++u) {
          const int sl = j0 + (int)threadIdx.x + u * kBlock;
          const bool ok = i >= 0 && sl < nsl;
          dw[r][u] = ld16z_nt(wd + (size_t)(ok ? i : 0) * rb + (size_t)sl * 16, ok);
        }
      }
    };
    // ---- up: one wave per row of the split, UN 16-byte slices per lane per pass
    const int step = UN * kWave * EPL;
    uint4 wu[UN], wg[UN];
    float uacc[NB], gacc[NB];
    int i = -1;
    size_t ro = 0;
    auto row_begin = [&](int kr) {
      i = kr < nr ? s_i[kr] : -1;
      ro = (size_t)(i >= 0 ? i : 0) * rb;
#pragma unroll
      for (int b = 0; b < NB; ++b) uacc[b] = gacc[b] = 0.f;
    };
    auto up_load = [&](int e0) {
#pragma unroll
      for (int q = 0; q < UN; ++q) {
        const int e = e0 + (q * kWave + lane) * EPL;
        const bool ok = i >= 0 && e < g.d;
        const size_t off = ro + (size_t)e * Tr<WT>::ESZ;
        wu[q] = ld16z_nt(reinterpret_cast<const char*>(g.w_up) + off, ok);
        if constexpr (ACT == PSFFN_SWIGLU) wg[q] = ld16z_nt(reinterpret_cast<const char*>(g.w_gate) + off, ok);
      }
    };
    auto up_acc = [&](int e0) {
#pragma unroll
      for (int q = 0; q < UN; ++q) {
        const int e = e0 + (q * kWave + lane) * EPL;
        const int ec = e < g.d ? e : 0;  // (the weights past d are zero)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < g.B) {
            const char* xr = xs + (size_t)b * g.d * XSZ;
            uacc[b] = dot16<WT>(wu[q], xr, ec, 1.f, uacc[b]);
            if constexpr (ACT == PSFFN_SWIGLU) gacc[b] = dot16<WT>(wg[q], xr, ec, 1.f, gacc[b]);
          }
      }
    };
    auto row_end = [&](int kr) {
      const bool valid = i >= 0;
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
        if (!valid || b >= g.B) av = 0.f;
        if (lane == 0 && kr < nr) s_a[kr * NB + b] = av;
      }
    };
    // the first row's first pass goes out before the first down batch, which then streams while
    // the up rows are reduced.  With several tokens (more arithmetic per row) and rows of one pass,
    // a wave requests its next row before it reduces the current one (a second register set).
    constexpr bool kDoubleRow = NB > 1;
    if (kDoubleRow && g.d <= step) {
      constexpr int NW = kBlock / kWave;
      uint4 nu_[kDoubleRow ? UN : 1], ng_[kDoubleRow ? UN : 1];
      int ni = -1;
      size_t nro = 0;
      auto next_load = [&](int kr) {
        ni = kr < nr ? s_i[kr] : -1;
        nro = (size_t)(ni >= 0 ? ni : 0) * rb;
#pragma unroll
        for (int q = 0; q < (kDoubleRow ? UN : 1); ++q) {
          const int e = (q * kWave + lane) * EPL;
          const bool ok = ni >= 0 && e < g.d;
          const size_t off = nro + (size_t)e * Tr<WT>::ESZ;
          nu_[q] = ld16z_nt(reinterpret_cast<const char*>(g.w_up) + off, ok);
          if constexpr (ACT == PSFFN_SWIGLU) ng_[q] = ld16z_nt(reinterpret_cast<const char*>(g.w_gate) + off, ok);
        }
      };
      auto take_next = [&]() {
        i = ni;
        ro = nro;
#pragma unroll
        for (int q = 0; q < (kDoubleRow ? UN : 1); ++q) {
          wu[q] = nu_[q];
          if constexpr (ACT == PSFFN_SWIGLU) wg[q] = ng_[q];
        }
      };
      row_begin(wv);
      up_load(0);
      load_down(0, 0);
      for (int k0 = 0; k0 < nr; k0 += NW) {
        next_load(k0 + NW + wv);  // (past the split: the zero block)
        up_acc(0);
        row_end(k0 + wv);
        if (k0 + NW >= nr) break;
#pragma unroll
        for (int b = 0; b < NB; ++b) uacc[b] = gacc[b] = 0.f;
        take_next();
      }
    } else {
      row_begin(wv);
      up_load(0);
      load_down(0, 0);
      up_acc(0);
      for (int e0 = step; e0 < g.d; e0 += step) {
        up_load(e0);
        up_acc(e0);
      }
      row_end(wv);
      for (int k0 = kBlock / kWave; k0 < nr; k0 += kBlock / kWave) {
        row_begin(k0 + wv);
        for (int e0 = 0; e0 < g.d; e0 += step) {
          up_load(e0);
          up_acc(e0);
        }
        row_end(k0 + wv);
      }
    }
    __syncthreads();
    // ---- down: thread t owns 16-byte column slices t + u kBlock; the next batch of RB rows is
    // requested before the current one is accumulated
    for (int j0 = 0; j0 < nsl; j0 += UG * kBlock) {
      if (j0 > 0) load_down(j0, 0);
      float acc[UG][NB][CPL];
#pragma unroll
      for (int u = 0; u < UG; ++u)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[u][b][c] = 0.f;
      for (int r0 = 0; r0 < nr; r0 += RB) {
        uint4 w[RB][UG];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int u = 0; u < UG; ++u) w[r][u] = dw[r][u];
        if (r0 + RB < nr) load_down(j0, r0 + RB);  // the next batch, if there is one
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (r0 + r >= nr) continue;  // (no break: the loop must unroll, w[r] stays in registers)
          float ab[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) ab[b] = s_a[(r0 + r) * NB + b];
#pragma unroll
          for (int u = 0; u < UG; ++u) {
            float wv8[CPL];
            if constexpr (WT == St::F32) {
              wv8[0] = __uint_as_float(w[r][u].x); wv8[1] = __uint_as_float(w[r][u].y);
              wv8[2] = __uint_as_float(w[r][u].z); wv8[3] = __uint_as_float(w[r][u].w);
            } else {
              const uint32_t ww[4] = {w[r][u].x, w[r][u].y, w[r][u].z, w[r][u].w};
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                wv8[2 * h] = h2f(ww[h] & 0xffffu);
                wv8[2 * h + 1] = h2f(ww[h] >> 16);
              }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
              for (int c = 0; c < CPL; ++c) acc[u][b][c] = fmaf(ab[b], wv8[c], acc[u][b][c]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        const int sl = j0 + (int)threadIdx.x + u * kBlock;
        if (sl >= nsl) continue;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b >= g.B) continue;
          float* dst = g.part + ((size_t)s * g.B + b) * g.d + (size_t)sl * CPL;
#pragma unroll
          for (int c = 0; c < CPL; c += 4)
            *reinterpret_cast<float4*>(dst + c) = make_float4(acc[u][b][c], acc[u][b][c + 1], acc[u][b][c + 2],
                                                              acc[u][b][c + 3]);
        }
      }
    }
    store_list();
  }
}

// y = (accumulate ? y : 0) + (b_down + the S split partials summed in split order).  Workgroup =
// kRQ float4 columns (4 kRQ consecutive outputs); its kRG thread groups take consecutive ranges
// of splits (at most 8 loads each in flight), and the group sums are added in group order.
constexpr int kRQ = 8;
constexpr int kRG = kBlock / kRQ;

template <St WT, psffn_act ACT>
__global__ __launch_bounds__(kBlock) void k_reduce_ud(FfnArgs g) {
  __shared__ float4 s_sum[kRG][kRQ];
  const int n = list_len(g.count, g.F);  // the layer path's up kernel wrote it
  int ks, S;
  udsplit<WT>(n, g.B, g.d, ud_stream_bytes<WT>(g.d, ACT), ks, S);
  const size_t total4 = (size_t)g.B * g.d / 4;
  const int q = threadIdx.x % kRQ, grp = threadIdx.x / kRQ;
  const size_t o4 = (size_t)blockIdx.x * kRQ + q;
  const int per = (S + kRG - 1) / kRG;
  const int s0 = grp * per, s1 = min(S, s0 + per);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (o4 < total4) {
    const float4* p = reinterpret_cast<const float4*>(g.part);
    for (int b0 = s0; b0 < s1; b0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b0 + u < s1 ? p[(size_t)(b0 + u) * total4 + o4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < s1) {
          acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
        }
    }
  }
  s_sum[grp][q] = acc;
  __syncthreads();
  if (grp == 0 && o4 < total4) {
    // y and b_down are only 4-byte aligned: scalar accesses
    const int col = (int)((o4 * 4) % (size_t)g.d);
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    if (g.b_down) {
#pragma unroll
      for (int c = 0; c < 4; ++c) t[c] = g.b_down[col + c];
    }
    for (int k = 0; k < kRG; ++k) {
      const float4 v = s_sum[k][q];
      t[0] += v.x; t[1] += v.y; t[2] += v.z; t[3] += v.w;
    }
    float* yp = g.y + o4 * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) yp[c] = g.accumulate ? yp[c] + t[c] : t[c];
  }
}

// =========================================================================================
// launchers

template <St PT, int NB, int RV>
static hipError_t predict_t(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx, int32_t* count,
                            float* logits, void* ws, hipStream_t s, int n_hot) {
  constexpr int RPW = 4;               // k_q chunks of 16 neurons
  const int NC = (P.F + 4 * RPW - 1) / (4 * RPW);
  const int NQ = (P.F + 31) / 32;      // 32-bit mask words
  if ((size_t)B * P.d * Tr<PT>::ESZ > (size_t)kStageX || NQ > kMaxScanChunks) return hipErrorNotSupported;
  const StateLayout L = state_layout(P.F);
  char* w = static_cast<char*>(ws);
  uint32_t* masks = reinterpret_cast<uint32_t*>(w + L.masks);
  float* h = reinterpret_cast<float*>(w + L.scratch);
  const size_t xbytes = round256((size_t)B * P.d * Tr<PT>::ESZ);
  // one token, fp16: k_h1 (one single-wave workgroup per row of A, the same h bits as k_h)
  const hipError_t eh = PT == St::F16 && B == 1 ? launch_h1(P, x, h, s) : hipErrorNotSupported;
  if (eh != hipSuccess && eh != hipErrorNotSupported) return eh;
  if (eh == hipErrorNotSupported)
    k_h<PT, NB, 0><<<(P.r + kHThreads / kWave - 1) / (kHThreads / kWave), kHThreads, xbytes, s>>>(P.A, x, P.d, P.r, B,
                                                                                               h, 0.f, nullptr);
  k_q<PT, NB, RV, RPW><<<NC, kBlock, 0, s>>>(P.Q, P.c, h, P.r, P.F, thr, B, logits, NC, masks, n_hot);
  k_list<<<1, kListThreads, 4 * (size_t)NQ, s>>>(masks, NQ, P.F, idx, count);
  return hipGetLastError();
}

// k_h alone at one token for an fp16 predictor: h = A x, or with ln.xres the LayerNorm of the fp32
// residual inside (its fp16 rows go to ln.hout) and h = A LN(x)
hipError_t launch_h_f16_b1(const psffn_predictor& P, const void* x, float* h, const LnArgs& ln, hipStream_t s,
                           uint32_t* zero, int nzero, uint32_t* zero2, int nzero2) {
  if (P.dt != PSFFN_F16 || (size_t)P.d * 2 > (size_t)kStageX) return hipErrorNotSupported;
  const size_t xbytes = round256((size_t)P.d * 2);
  const int hgrid = (P.r + kHThreads / kWave - 1) / (kHThreads / kWave);
  if (ln.xres == nullptr) {
    k_h<St::F16, 1, 0><<<hgrid, kHThreads, xbytes, s>>>(P.A, x, P.d, P.r, 1, h, 0.f, nullptr, zero, nzero, zero2, nzero2);
  } else {
    const int k = ln_k(P.d);
    if (k == 1) k_h<St::F16, 1, 1><<<hgrid, kHThreads, xbytes, s>>>(P.A, ln.xres, P.d, P.r, 1, h, ln.eps, ln.hout, zero, nzero, zero2, nzero2);
    else if (k == 2) k_h<St::F16, 1, 2><<<hgrid, kHThreads, xbytes, s>>>(P.A, ln.xres, P.d, P.r, 1, h, ln.eps, ln.hout, zero, nzero, zero2, nzero2);
    else if (k == 4) k_h<St::F16, 1, 4><<<hgrid, kHThreads, xbytes, s>>>(P.A, ln.xres, P.d, P.r, 1, h, ln.eps, ln.hout, zero, nzero, zero2, nzero2);
    else if (k == 8) k_h<St::F16, 1, 8><<<hgrid, kHThreads, xbytes, s>>>(P.A, ln.xres, P.d, P.r, 1, h, ln.eps, ln.hout, zero, nzero, zero2, nzero2);
    else if (k == 16) k_h<St::F16, 1, 16><<<hgrid, kHThreads, xbytes, s>>>(P.A, ln.xres, P.d, P.r, 1, h, ln.eps, ln.hout, zero, nzero, zero2, nzero2);
    else return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <St PT, int NB>
static hipError_t predict_rv(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx, int32_t* count,
                             float* logits, void* ws, hipStream_t s, int n_hot) {
  const int per = kWave * Tr<PT>::EPL;  // elements of a row covered by one 16-byte slice per lane
  const int rv = (P.r + per - 1) / per;
  if (rv == 1) return predict_t<PT, NB, 1>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  if (rv == 2) return predict_t<PT, NB, 2>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  if (rv == 3) return predict_t<PT, NB, 3>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  if (rv == 4) return predict_t<PT, NB, 4>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  return hipErrorNotSupported;
}

template <St PT>
static hipError_t predict_nb(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx, int32_t* count,
                             float* logits, void* ws, hipStream_t s, int n_hot) {
  if (B == 1) return predict_rv<PT, 1>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  if (B == 2) return predict_rv<PT, 2>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  if (B <= 4) return predict_rv<PT, 4>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  return hipErrorNotSupported;
}

hipError_t launch_predict_fused(St st, const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx,
                                int32_t* count, float* logits, void* ws, hipStream_t s, int n_hot) {
  if (st == St::F32) return predict_nb<St::F32>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  if (st == St::F16) return predict_nb<St::F16>(P, x, B, thr, idx, count, logits, ws, s, n_hot);
  return hipErrorNotSupported;
}

template <St WT>
static bool ffn_fits(const psffn_ffn& W, int B) {
  // every split fits the fused kernel's row capacity, x fits LDS
  return W.F <= kUDSplitCap * kUDMaxRows && (size_t)B * W.d * (WT == St::F32 ? 4 : 2) <= (size_t)kStageX;
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
  g.y = y;
  g.B = B;
  g.d = W.d;
  g.F = W.F;
  g.accumulate = accumulate;
  g.xbytes = round256((size_t)B * W.d * (WT == St::F32 ? 4 : 2));
  return g;
}

template <St WT, psffn_act ACT, int NB, bool SCAN>
static size_t ud_lds(const FfnArgs& g) {
  return g.xbytes + (SCAN ? round256(4 * (size_t)(2 * g.nq + 1)) : 0) + 4 * (size_t)kUDMaxRows * NB +
         4 * (size_t)kUDMaxRows;
}

template <St WT, psffn_act ACT, int NB, bool SCAN>
static hipError_t ud_attr() {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ud<WT, ACT, NB, SCAN>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
  return e;
}

template <St WT, psffn_act ACT, int NB, bool SCAN>
static hipError_t ffn_launch(const FfnArgs& g, hipStream_t s) {
  const size_t lds = ud_lds<WT, ACT, NB, SCAN>(g);
  if (lds > (size_t)64 * 1024) {
    const hipError_t e = ud_attr<WT, ACT, NB, SCAN>();
    if (e != hipSuccess) return e;
  }
  int grid = kUDSplitCap;
  if (grid > g.F) grid = g.F;
  k_ud<WT, ACT, NB, SCAN><<<grid, kBlock, lds, s>>>(g);
  k_reduce_ud<WT, ACT><<<(unsigned)(((size_t)g.B * g.d / 4 + kRQ - 1) / kRQ), kBlock, 0, s>>>(g);
  return hipGetLastError();
}

template <St WT, psffn_act ACT, int NB>
static hipError_t ffn_t(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count, float* y,
                        int accumulate, void* ws, hipStream_t s) {
  if (!ffn_fits<WT>(W, B)) return hipErrorNotSupported;
  return ffn_launch<WT, ACT, NB, false>(ffn_args<WT>(W, x, B, idx, count, y, accumulate, ws), s);
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

// ---- the FFN from mask words already in the workspace: k_ud in scan mode (orders the list from the
// masks, writes idx/count, the activations and the down-projection partials), k_reduce_ud

template <St WT, psffn_act ACT, int NB>
static hipError_t ffn_scan_t(const psffn_ffn& W, const void* x, int B, int32_t* idx, int32_t* count, float* y,
                             int accumulate, void* ws, hipStream_t s, int n_hot) {
  const int NQ = (W.F + 31) / 32;
  const size_t ud = round256((size_t)B * W.d * (WT == St::F32 ? 4 : 2)) + round256(4 * (size_t)(2 * NQ + 1)) +
                    4 * (size_t)kUDMaxRows * NB + 4 * (size_t)kUDMaxRows;
  if (!ffn_fits<WT>(W, B) || NQ > kMaxScanChunks || ud > (size_t)150 * 1024) return hipErrorNotSupported;
  FfnArgs g = ffn_args<WT>(W, x, B, idx, count, y, accumulate, ws);
  g.masks = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + state_layout(W.F).masks);
  g.nq = NQ;
  g.idx_out = idx;
  g.count_out = count;
  g.n_hot = n_hot;
  return ffn_launch<WT, ACT, NB, true>(g, s);
}

template <St WT, psffn_act ACT>
static hipError_t ffn_scan_nb(const psffn_ffn& W, const void* x, int B, int32_t* idx, int32_t* count, float* y,
                              int accumulate, void* ws, hipStream_t s, int n_hot) {
  if (B == 1) return ffn_scan_t<WT, ACT, 1>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
  if (B == 2) return ffn_scan_t<WT, ACT, 2>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
  if (B <= 4) return ffn_scan_t<WT, ACT, 4>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
  return hipErrorNotSupported;
}

bool ffn_fused_scan_fits(const psffn_ffn& W, int B) {
  if (B < 1 || B > kFusedMaxBatch) return false;
  const int NB = B == 1 ? 1 : (B == 2 ? 2 : 4);
  const int NQ = (W.F + 31) / 32;
  const size_t xe = W.dt == PSFFN_F32 ? 4 : 2;
  const size_t ud = round256((size_t)B * W.d * xe) + round256(4 * (size_t)(2 * NQ + 1)) +
                    4 * (size_t)kUDMaxRows * NB + 4 * (size_t)kUDMaxRows;
  return W.F <= kUDSplitCap * kUDMaxRows && (size_t)B * W.d * xe <= (size_t)kStageX && NQ <= kMaxScanChunks &&
         ud <= (size_t)150 * 1024;
}

hipError_t launch_ffn_fused_scan(St st, const psffn_ffn& W, const void* x, int B, int32_t* idx, int32_t* count,
                                 float* y, int accumulate, void* ws, hipStream_t s, int n_hot) {
  if (W.act == PSFFN_RELU) {
    if (st == St::F32) return ffn_scan_nb<St::F32, PSFFN_RELU>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
    if (st == St::F16) return ffn_scan_nb<St::F16, PSFFN_RELU>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
    return ffn_scan_nb<St::I4, PSFFN_RELU>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
  }
  if (st == St::F32) return ffn_scan_nb<St::F32, PSFFN_SWIGLU>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
  if (st == St::F16) return ffn_scan_nb<St::F16, PSFFN_SWIGLU>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
  return ffn_scan_nb<St::I4, PSFFN_SWIGLU>(W, x, B, idx, count, y, accumulate, ws, s, n_hot);
}

// ---- one decode step of one layer: k_h, k_q (mask words only), then the FFN from the mask words

template <St PT, St WT, psffn_act ACT, int NB, int RV>
static hipError_t layer_t(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr, int32_t* idx,
                          int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s,
                          int n_hot, const LnArgs& ln) {
  const float* xres = ln.xres;
  const float eps = ln.eps;
  _Float16* hout = ln.hout;
  constexpr int RPW = 4;                  // k_q chunks of 16 neurons (32 KB of Q rows in flight each)
  const int NQ = (P.F + 31) / 32;         // 32-bit mask words
  const int NC = (P.F + 4 * RPW - 1) / (4 * RPW);
  // the fused up/down kernel's LDS: the activations, the mask words and the split's rows
  const size_t ud = round256((size_t)B * W.d * (WT == St::F32 ? 4 : 2)) + round256(4 * (size_t)(2 * NQ + 1)) +
                    4 * (size_t)kUDMaxRows * NB + 4 * (size_t)kUDMaxRows;
  if (!ffn_fits<WT>(W, B) || NQ > kMaxScanChunks || (size_t)B * P.d * Tr<PT>::ESZ > (size_t)kStageX ||
      ud > (size_t)150 * 1024)
    return hipErrorNotSupported;
  const StateLayout L = state_layout(P.F);
  char* w = static_cast<char*>(ws);
  uint32_t* masks = reinterpret_cast<uint32_t*>(w + L.masks);
  float* h = reinterpret_cast<float*>(w + L.scratch);
  const size_t xbytes = round256((size_t)B * P.d * Tr<PT>::ESZ);
  const int hgrid = (P.r + kHThreads / kWave - 1) / (kHThreads / kWave);
  if (xres == nullptr) {
    // one token, fp16: k_h1, as in the predictor call (the same h bits as k_h)
    const hipError_t eh = PT == St::F16 && B == 1 ? launch_h1(P, x, h, s) : hipErrorNotSupported;
    if (eh != hipSuccess && eh != hipErrorNotSupported) return eh;
    if (eh == hipErrorNotSupported) k_h<PT, NB, 0><<<hgrid, kHThreads, xbytes, s>>>(P.A, x, P.d, P.r, B, h, 0.f, nullptr);
  } else {
    if constexpr (PT != St::F16) return hipErrorNotSupported;
    else {
      const int k = ln_k(P.d);
      if (k == 1) k_h<PT, NB, 1><<<hgrid, kHThreads, xbytes, s>>>(P.A, xres, P.d, P.r, B, h, eps, hout);
      else if (k == 2) k_h<PT, NB, 2><<<hgrid, kHThreads, xbytes, s>>>(P.A, xres, P.d, P.r, B, h, eps, hout);
      else if (k == 4) k_h<PT, NB, 4><<<hgrid, kHThreads, xbytes, s>>>(P.A, xres, P.d, P.r, B, h, eps, hout);
      else if (k == 8) k_h<PT, NB, 8><<<hgrid, kHThreads, xbytes, s>>>(P.A, xres, P.d, P.r, B, h, eps, hout);
      else if (k == 16) k_h<PT, NB, 16><<<hgrid, kHThreads, xbytes, s>>>(P.A, xres, P.d, P.r, B, h, eps, hout);
      else return hipErrorNotSupported;
    }
  }
  k_q<PT, NB, RV, RPW><<<NC, kBlock, 0, s>>>(P.Q, P.c, h, P.r, P.F, thr, B, logits, NC, masks, n_hot);
  return ffn_scan_t<WT, ACT, NB>(W, xres ? static_cast<const void*>(hout) : x, B, idx, count, y, accumulate, ws, s,
                                 n_hot);
}

template <St PT, St WT, psffn_act ACT, int NB>
static hipError_t layer_rv(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr, int32_t* idx,
                           int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s,
                           int n_hot, const LnArgs& ln) {
  const int per = kWave * Tr<PT>::EPL;
  const int rv = (P.r + per - 1) / per;
  if (rv == 1) return layer_t<PT, WT, ACT, NB, 1>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  if (rv == 2) return layer_t<PT, WT, ACT, NB, 2>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  if (rv == 3) return layer_t<PT, WT, ACT, NB, 3>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  if (rv == 4) return layer_t<PT, WT, ACT, NB, 4>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  return hipErrorNotSupported;
}

template <St PT, St WT, psffn_act ACT>
static hipError_t layer_nb(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr, int32_t* idx,
                           int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s,
                           int n_hot, const LnArgs& ln) {
  if (B == 1) return layer_rv<PT, WT, ACT, 1>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  if (B == 2) return layer_rv<PT, WT, ACT, 2>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  if (B <= 4) return layer_rv<PT, WT, ACT, 4>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  return hipErrorNotSupported;
}

template <St PT, St WT>
static hipError_t layer_act(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                            int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                            hipStream_t s, int n_hot, const LnArgs& ln) {
  if (W.act == PSFFN_RELU)
    return layer_nb<PT, WT, PSFFN_RELU>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  return layer_nb<PT, WT, PSFFN_SWIGLU>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
}

hipError_t launch_layer_fused(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                              int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                              hipStream_t s, int n_hot, const LnArgs& ln) {
  if (P.dt == PSFFN_F32 && W.dt == PSFFN_F32) {
    if (ln.xres) return hipErrorNotSupported;
    return layer_act<St::F32, St::F32>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  }
  if (P.dt == PSFFN_F16 && W.dt == PSFFN_F16)
    return layer_act<St::F16, St::F16>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  if (P.dt == PSFFN_F16 && W.dt == PSFFN_I4G128)
    return layer_act<St::F16, St::I4>(P, W, x, B, thr, idx, count, logits, y, accumulate, ws, s, n_hot, ln);
  return hipErrorNotSupported;
}

}  // namespace psffn

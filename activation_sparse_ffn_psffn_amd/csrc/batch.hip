// Batch pipeline (4 < B <= 32; fp16 predictor, fp16 or 4-bit FFN weights) on MFMA tiles.
//
// With several tokens every weight element is used B times, which a wave can no longer feed
// from its vector ALUs at HBM rate (B fp32 FMAs per 2-byte weight); matrix cores take the
// products instead.  Every contraction is a v_mfma_f32_16x16x32_f16 over 16 weight rows (or
// columns) x 16 tokens (the batch is padded to NBP = 16 or 32 token columns with zeros):
//
//   k_bh      partial h over 512-element chunks of d            h = A x          (16 rows / wave)
//   k_bhred   h = sum of the chunks in chunk order, split into fp16 hi + lo parts
//   k_bq_lds  logits Q (h_hi + h_lo) + c, union test over the batch, one mask word per 32 neurons
//             (h in LDS; k_bq reads it from L2 when it does not fit)
//   k_bscan   the ascending list and its length from the mask words (one workgroup)
//   k_bup     up (and gate) rows of 64 listed neurons x one chunk of d; x staged in LDS
//   k_bact    pre-activations summed over the chunks in chunk order, bias, ReLU / SiLU-gate
//   k_bdown   column tiles x row splits of sum_k a_k W_dT[idx[k]], transposed through LDS
//   k_breduce y = b_down + the split partials in split order (+ y when accumulating)
//
// Method ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur
// Research summary): Summary 2nd paragraph (per-layer predictor, neuron-level kernels that skip
// the inactive neurons) and Interesting ideas I4 (whole rows and columns, no sparse format); a
// batch shares the union of its tokens' predicted sets.
//
// Precision: weights and activations are fp16 (or exact small integers for 4-bit weights), so
// every product is exact in the fp32 accumulator.  The fp32 values that feed a contraction (h for
// the logits, the activations for the down projection) are split as v = hi + lo with hi, lo
// fp16, which keeps 22 significant bits, and both halves are multiplied: the logits and outputs
// stay at fp32 accuracy.
//
// MFMA operand layout (16x16x32, fp16; lane L, i = L % 16, g = L / 16): the A operand of lane L
// holds A[i][8g .. 8g+8), the B operand B[8g .. 8g+8)[i], and the result D[4g + v][i], v < 4.
// The k index of a contraction is free to permute as long as both operands agree; over d the
// kernels use "block of 128, lane group g owns elements [32g, 32g+32), step s uses
// [32g + 8s, 32g + 8s + 8)", so each lane reads 64 contiguous bytes of a row per block (16
// bytes for 4-bit rows: one word of 8 nibbles per step).
#include "common.h"

namespace psffn {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4_t mma(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h8_t as_h8(uint4 v) { return __builtin_bit_cast(h8_t, v); }
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// Buffer loads (MUBUF): a resource holds the base and the byte size of an array, the lane gives a
// 32-bit byte offset, and a read past the size returns zeros in hardware.  One VGPR of address per
// lane instead of two, no predicate, and an out-of-range row reads as zeros.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
// The weight loads here keep the default cache policy: an MFMA fragment layout splits each 128-byte
// line of a weight row over several load instructions and waves, and marked non-temporal such lines
// were fetched again (measured on MI355X: OPT-175B-shaped 4-bit layer at 8 tokens 102.7 -> 133.3 us,
// 48-layer stack at 4 tokens 1353 -> 1040 tokens/s), unlike the one-token kernels, whose loads take
// whole lines in one instruction.
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// An offset past every buffer (the load returns zeros).  Buffers are kept below 2 GiB, so
// kNoRow plus any in-row offset (< 2 GiB) neither wraps nor lands inside a buffer.
constexpr uint32_t kNoRow = 0x80000000u;
constexpr size_t kMaxBufferBytes = (size_t)0x7FFFFFFF;

// Loads that are issued whatever the predicate: when it is false they read a block of zeros in
// device memory instead.  No branch around the load and no select after it, so the compiler's
// wait counting stays exact and a ring of loads in flight is not drained at every step.
__device__ uint4 g_zero16[1] = {{0u, 0u, 0u, 0u}};  // never written

__device__ __forceinline__ uint4 ld16_or0(const void* p, bool ok, const void*) {
  return ldg16(ok ? p : static_cast<const void*>(g_zero16));
}
__device__ __forceinline__ uint32_t ld16b_or0(const uint16_t* p, bool ok, const uint16_t*) {
  return (uint32_t)*(ok ? p : reinterpret_cast<const uint16_t*>(g_zero16));
}

// A operand from one word of 8 nibbles e0..e7: [e0 e4 e1 e5 e2 e6 e3 e7] (exact small integers);
// the activations are paired the same way by pair_x8.
__device__ __forceinline__ h8_t i4_frag(uint32_t w) {
  const half2_t p0 = i4_pair(w, 0), p1 = i4_pair(w, 4), p2 = i4_pair(w, 8), p3 = i4_pair(w, 12);
  h8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// v = hi + lo, hi = fp16(v), lo = fp16(v - hi)
__device__ __forceinline__ void split_hl(float v, _Float16& hi, _Float16& lo) {
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

constexpr int kHChunk = 512;       // elements of d per partial h
constexpr int kBatchMaxF = 98304;  // the up kernel's LDS (x chunk + list scan) stays under 64 KB
constexpr int kBSplitCap = 16;      // max row splits of the down projection
constexpr int kDPitch = 136;        // LDS bytes per row of a wave's 32 x 64 fp16 weight block

// ---- arguments -------------------------------------------------------------------------------
struct BArgs {
  // predictor
  const uint16_t* A;
  const uint16_t* Q;
  const float* c;
  int r;
  float thr;
  float* logits;
  float* hpart;
  uint16_t* hhi;
  uint16_t* hlo;
  uint32_t* masks;
  int nq;
  int n_hot;  // hot prefix: neurons [0, n_hot) are listed whatever their logits
  int32_t* idx_out;
  int32_t* count_out;
  // shared
  const uint16_t* x;
  int B, d, F;
  // FFN
  const void* w_up;
  const void* w_gate;
  const void* w_dT;
  const uint16_t* s_up;
  const uint16_t* s_gate;
  const uint16_t* s_dT;
  const float* b_up;
  const float* b_gate;
  const float* b_down;
  const int32_t* idx;
  const int32_t* count;
  float* upart;
  float* gpart;
  int ldk;  // row stride (neurons) of the per-token activation arrays: F rounded up to 32
  float* aT;
  uint16_t* ahi;
  uint16_t* alo;
  float* part;
  float* y;
  int accumulate;
};

__device__ __forceinline__ int blist_len(const int32_t* count, int F) {
  const int n = *count;
  return n < 0 ? 0 : (n > F ? F : n);
}

// Row splits of the down projection for a list of n neurons: at least enough splits for each to
// fit one chunk of the down kernel, more while the partials (S x B x d fp32) stay below about a
// quarter of the weight bytes the splits stream, at most kBSplitCap; each split is a whole number
// of 32-row steps.  S >= 1 (an empty list still writes one zero partial).
__device__ __forceinline__ void bsplit(int n, int B, int d, int row_bytes, int chunk_rows, int& ks, int& S) {
  long long want = (long long)n * row_bytes / ((long long)B * d * 16);
  const long long fit = (n + chunk_rows - 1) / chunk_rows;  // splits of at most one chunk, if allowed
  if (want < fit) want = fit;
  if (want < 1) want = 1;
  if (want > kBSplitCap) want = kBSplitCap;
  ks = (int)((n + want - 1) / want);
  ks = (ks + 31) & ~31;
  if (ks < 32) ks = 32;
  S = n > 0 ? (n + ks - 1) / ks : 1;
}

// ---- list ordering from mask words (bit b of word q: neuron 32q + b is active) ----------------
template <int NTH>
__device__ void mask_prefix(const uint32_t* __restrict__ masks, int nq, int n_hot, uint32_t* s_mask, int* s_pre,
                            int* s_red) {
  for (int q0 = threadIdx.x; q0 < nq; q0 += 8 * NTH) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = q0 + u * NTH < nq ? masks[q0 + u * NTH] : 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + u * NTH;
      // the hot prefix's bits (n_hot <= F, so no bit past F is set)
      const int nh = n_hot - 32 * q;
      const uint32_t hot = nh >= 32 ? 0xffffffffu : (nh > 0 ? (1u << nh) - 1u : 0u);
      if (q < nq) s_mask[q] = v[u] | hot;
    }
  }
  __syncthreads();
  const int per = (nq + NTH - 1) / NTH;  // consecutive words per thread
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
  int run = inc - tot;
  for (int w = 0; w < wv; ++w) run += s_red[w];
  for (int u = 0; u < per; ++u)
    if (q0 + u < nq) {
      s_pre[q0 + u] = run;
      run += __popc(s_mask[q0 + u]);
    }
  if (threadIdx.x == NTH - 1) s_pre[nq] = run;
  __syncthreads();
}

// The neuron at list position k (0 <= k < total): the last word q whose prefix count is <= k holds
// it, as its (k - s_pre[q])-th set bit.
__device__ __forceinline__ int list_at(const uint32_t* s_mask, const int* s_pre, int nq, int k) {
  int lo = 0, hi = nq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  uint32_t m = s_mask[lo];
  for (int j = k - s_pre[lo]; j > 0; --j) m &= m - 1u;
  return lo * 32 + (int)__builtin_ctz(m);
}

// =============================================================================================
// k_bh: wave (row tile rt, chunk kc): partial h over d-elements [512 kc, 512 kc + 512) of rows
// [16 rt, 16 rt + 16).  Grid (ceil(d / 512), ceil(r / 64)): consecutive workgroups read consecutive
// chunks of the same 64 rows.  Each wave requests its 16 A fragments first (buffer loads: rows
// past r and columns past d read zeros), then the workgroup stages the chunk of x (all padded
// token rows) in LDS once; the MFMAs read their x fragments from there.  One memory round trip
// per wave.  hpart[kc][n][j], n < NBP (padded tokens give zeros).

template <int NT>
__global__ __launch_bounds__(kBlock) void k_bh(BArgs g) {
  constexpr int NBP = 16 * NT;
  constexpr int XP = kHChunk + 8;  // LDS pitch (elements): rows 16 bytes apart in bank order
  __shared__ __align__(16) uint16_t s_xc[NBP * XP];
  const int lane = wave_lane(), li = lane & 15, lg = lane >> 4;
  const int rt = blockIdx.y * 4 + wave_id();
  const int kc = blockIdx.x;
  const int d = g.d;
  const __amdgpu_buffer_rsrc_t ar = rsrc(g.A, (uint32_t)((size_t)g.r * d * 2));
  const __amdgpu_buffer_rsrc_t xr = rsrc(g.x, (uint32_t)((size_t)g.B * d * 2));
  const int row = rt * 16 + li;
  const uint32_t rbase = row < g.r ? (uint32_t)((size_t)row * d * 2) : kNoRow;
  uint4 w[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = kc * kHChunk + (j >> 2) * 128 + lg * 32 + (j & 3) * 8;
    w[j] = bld16(ar, e < d ? rbase + (uint32_t)e * 2 : kNoRow);
  }
  {
    constexpr int PIECES = NBP * (kHChunk / 8);  // 16-byte pieces of the x chunk
    constexpr int PPT = PIECES / kBlock;
    static_assert(PIECES % kBlock == 0, "whole pieces per thread");
    uint4 xv[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pc = threadIdx.x + k * kBlock;
      const int n = pc / (kHChunk / 8), e = kc * kHChunk + (pc % (kHChunk / 8)) * 8;
      xv[k] = bld16(xr, (n < g.B && e < d) ? (uint32_t)((size_t)n * d + e) * 2 : kNoRow);
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pc = threadIdx.x + k * kBlock;
      const int n = pc / (kHChunk / 8), e8 = pc % (kHChunk / 8);
      *reinterpret_cast<uint4*>(&s_xc[n * XP + e8 * 8]) = xv[k];
    }
  }
  __syncthreads();
  if (rt * 16 >= g.r) return;
  f4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int el = (j >> 2) * 128 + lg * 32 + (j & 3) * 8;  // element within the chunk
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint4 xf = *reinterpret_cast<const uint4*>(&s_xc[(t * 16 + li) * XP + el]);
      acc[t] = mma(as_h8(w[j]), as_h8(xf), acc[t]);
    }
  }
  const int j0 = rt * 16 + 4 * lg;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float* dst = g.hpart + ((size_t)kc * (16 * NT) + t * 16 + li) * g.r + j0;
    if (j0 + 3 < g.r) {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (j0 + v < g.r) dst[v] = acc[t][v];
    }
  }
}

// k_bhred: h[n][j] = sum over chunks in chunk order; hi/lo fp16 parts [NBP][r] (zero for n >= B)
__global__ __launch_bounds__(kBlock) void k_bhred(BArgs g, int ksh, int nbp) {
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= nbp * g.r) return;
  const int n = t / g.r;
  float s = 0.f;
  if (n < g.B) {
    constexpr int kR = 32;  // chunk partials in flight per round (one round up to d = 16384)
    for (int k0 = 0; k0 < ksh; k0 += kR) {
      float v[kR];
#pragma unroll
      for (int u = 0; u < kR; ++u) v[u] = k0 + u < ksh ? g.hpart[(size_t)(k0 + u) * nbp * g.r + t] : 0.f;
#pragma unroll
      for (int u = 0; u < kR; ++u)
        if (k0 + u < ksh) s += v[u];
    }
  }
  _Float16 hi, lo;
  split_hl(s, hi, lo);
  g.hhi[t] = __builtin_bit_cast(uint16_t, hi);
  g.hlo[t] = __builtin_bit_cast(uint16_t, lo);
}

// =============================================================================================
// k_bq: wave u covers neurons [32u, 32u + 32) (two row tiles) over all of r, blocks of 128
// software-pipelined (the next block's Q rows and h fragments are requested before the current
// block's MFMAs).  Writes mask word u and, optionally, the logits.

template <int NT>
__global__ __launch_bounds__(kBlock) void k_bq(BArgs g) {
  const int lane = wave_lane(), li = lane & 15, lg = lane >> 4;
  const int u = blockIdx.x * 4 + wave_id();
  if (u * 32 >= g.F) return;
  const int r = g.r;
  const int nkb = (r + 127) / 128;
  const uint16_t* qrow[2];
  bool qok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = u * 32 + t * 16 + li;
    qok[t] = i < g.F;
    qrow[t] = g.Q + (size_t)(qok[t] ? i : 0) * r;
  }
  uint4 qc[2][4], hc[NT][4], lc[NT][4];
  uint4 qn[2][4], hn[NT][4], ln[NT][4];
  auto load = [&](int kb, uint4 (&q)[2][4], uint4 (&hh)[NT][4], uint4 (&hl)[NT][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = kb * 128 + lg * 32 + s * 8;
      const bool in = e < r;
#pragma unroll
      for (int t = 0; t < 2; ++t) q[t][s] = (in && qok[t]) ? ldg16(qrow[t] + e) : zero4();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const size_t o = (size_t)(t * 16 + li) * r + e;
        hh[t][s] = in ? ldg16(g.hhi + o) : zero4();
        hl[t][s] = in ? ldg16(g.hlo + o) : zero4();
      }
    }
  };
  f4_t acc[2][NT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[a][t] = f4_t{0.f, 0.f, 0.f, 0.f};
  load(0, qc, hc, lc);
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load(kb + 1, qn, hn, ln);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[a][t] = mma(as_h8(qc[a][s]), as_h8(hc[t][s]), acc[a][t]);
          acc[a][t] = mma(as_h8(qc[a][s]), as_h8(lc[t][s]), acc[a][t]);
        }
    if (kb + 1 < nkb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int a = 0; a < 2; ++a) qc[a][s] = qn[a][s];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          hc[t][s] = hn[t][s];
          lc[t][s] = ln[t][s];
        }
      }
    }
  }
  uint32_t word = 0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = u * 32 + a * 16 + 4 * lg + v;
      const float ci = i < g.F ? g.c[i] : 0.f;
      unsigned long long any = 0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = t * 16 + li;
        const float l = acc[a][t][v] + ci;
        const bool ok = n < g.B && i < g.F;
        if (g.logits && ok) g.logits[(size_t)n * g.F + i] = l;
        any |= __ballot(ok && l > g.thr);
      }
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        if ((any >> (16 * gg)) & 0xffffull) word |= 1u << (a * 16 + 4 * gg + v);
    }
  if (lane == 0) g.masks[u] = word;
}

// k_bq_lds: the same result as k_bq with h (hi and lo, all NBP token rows) staged once per
// workgroup in LDS (up to 160 KB on gfx950); one workgroup of 8 waves per CU, each wave takes
// units of 32 neurons and keeps kBqRing blocks of Q rows in flight (a ring of registers refilled
// as each block is consumed), so a wave waits for HBM once per unit, not once per block.

constexpr int kBqThreads = 512;
constexpr int kBqRing = 4;

__host__ __device__ inline int bq_pitch(int r) { return 2 * r + 16; }  // LDS bytes per token row

template <int NT>
__global__ __launch_bounds__(kBqThreads) void k_bq_lds(BArgs g) {
  constexpr int NBP = 16 * NT;
  constexpr int D = kBqRing;
  extern __shared__ uint4 s_dyn4[];
  char* s_hi = reinterpret_cast<char*>(s_dyn4);
  const int r = g.r, hp = bq_pitch(r);
  char* s_lo = s_hi + NBP * hp;
  const int lane = wave_lane(), li = lane & 15, lg = lane >> 4;
  const int nwaves = gridDim.x * (kBqThreads / kWave);
  const int nunits = (g.F + 31) / 32;
  const int nkb = (r + 127) / 128;
  int u = blockIdx.x * (kBqThreads / kWave) + wave_id();
  uint4 q[D][2][4];
  auto loadq = [&](int uu, int kb, uint4(&qq)[2][4]) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int i = uu * 32 + a * 16 + li;
      const uint16_t* qr = g.Q + (size_t)(i < g.F ? i : 0) * r;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = kb * 128 + lg * 32 + s * 8;
        qq[a][s] = ld16_or0(qr + e, i < g.F && e < r, g.Q);
      }
    }
  };
  // the first unit's Q blocks go out before h is staged (block indices clamped to the last one)
  if (u < nunits) {
#pragma unroll
    for (int p = 0; p < D; ++p) loadq(u, p < nkb ? p : nkb - 1, q[p]);
  }
  {
    const int per_row = r / 8;  // 16-byte pieces per token row
    const int pieces = 2 * NBP * per_row;
    for (int p0 = threadIdx.x; p0 < pieces; p0 += 8 * kBqThreads) {
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int pc = p0 + k * kBqThreads;
        const int part = pc / (NBP * per_row), rem = pc % (NBP * per_row);
        const uint16_t* src = part == 0 ? g.hhi : g.hlo;
        v[k] = ld16_or0(src + (size_t)rem * 8, pc < pieces, nullptr);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int pc = p0 + k * kBqThreads;
        if (pc < pieces) {
          const int part = pc / (NBP * per_row), rem = pc % (NBP * per_row);
          const int n = rem / per_row, e8 = rem % per_row;
          *reinterpret_cast<uint4*>((part == 0 ? s_hi : s_lo) + n * hp + e8 * 16) = v[k];
        }
      }
    }
  }
  __syncthreads();
  for (; u < nunits; u += nwaves) {
    f4_t acc[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[a][t] = f4_t{0.f, 0.f, 0.f, 0.f};
    // one 128-wide block of Q rows against h from LDS (Q row elements past r are zero)
    auto block = [&](int kb, const uint4(&qq)[2][4]) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = kb * 128 + lg * 32 + s * 8;
        const int ec = e < r ? e : 0;
        uint4 hh[NT], hl[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int o = (t * 16 + li) * hp + ec * 2;
          hh[t] = *reinterpret_cast<const uint4*>(s_hi + o);
          hl[t] = *reinterpret_cast<const uint4*>(s_lo + o);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[a][t] = mma(as_h8(qq[a][s]), as_h8(hh[t]), acc[a][t]);
            acc[a][t] = mma(as_h8(qq[a][s]), as_h8(hl[t]), acc[a][t]);
          }
      }
    };
    // main groups: every block consumed refills its slot with the block D later (clamped)
    int kb0 = 0;
    for (; kb0 + D < nkb; kb0 += D) {
#pragma unroll
      for (int p = 0; p < D; ++p) {
        block(kb0 + p, q[p]);
        const int nx = kb0 + p + D;
        loadq(u, nx < nkb ? nx : nkb - 1, q[p]);
      }
    }
    // last group: no refills
#pragma unroll
    for (int p = 0; p < D; ++p)
      if (kb0 + p < nkb) block(kb0 + p, q[p]);
    uint32_t word = 0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = u * 32 + a * 16 + 4 * lg + v;
        const float ci = i < g.F ? g.c[i] : 0.f;
        unsigned long long any = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = t * 16 + li;
          const float l = acc[a][t][v] + ci;
          const bool ok = n < g.B && i < g.F;
          if (g.logits && ok) g.logits[(size_t)n * g.F + i] = l;
          any |= __ballot(ok && l > g.thr);
        }
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
          if ((any >> (16 * gg)) & 0xffffull) word |= 1u << (a * 16 + 4 * gg + v);
      }
    if (lane == 0) g.masks[u] = word;
    if (u + nwaves < nunits) {
#pragma unroll
      for (int p = 0; p < D; ++p) loadq(u + nwaves, p < nkb ? p : nkb - 1, q[p]);
    }
  }
}

// k_bq_full: as k_bq_lds, but a wave takes one row tile (16 neurons) at a time and requests all
// of its Q rows at once (NKB blocks of 128, 16 full rows in flight: the DRAM pages of a tile are
// read together), then runs the MFMAs against h in LDS.  h is stored zero-padded to NKB x 128
// elements per token, so the Q bytes read past a row's end (the next row, or zeros past the
// array) multiply zeros.  Writes the 16-bit half of the tile's mask word.

__host__ __device__ inline int bq_full_pitch(int nkb) { return nkb * 256 + 16; }

// one workgroup per CU (h in LDS).  16 tokens: four waves (at most 4 row tiles, <= 192 KB, in
// flight per CU: measured 32.5 us against 38.5 with eight on a 49152 x 1536 Q); 32 tokens: eight
// waves (twice the MFMA work per tile: 20.0 us against 21.6 with four on 32768 x 1024)
template <int NT>
__host__ __device__ constexpr int bq_full_threads() { return NT == 1 ? 256 : 512; }

template <int NT, int NKB>
__global__ __launch_bounds__(bq_full_threads<NT>()) void k_bq_full(BArgs g) {
  constexpr int kBqFullThreads = bq_full_threads<NT>();
  constexpr int NBP = 16 * NT;
  constexpr int HP = NKB * 256 + 16;
  constexpr int WPG = kBqFullThreads / kWave;
  extern __shared__ uint4 s_dyn4[];
  char* s_hi = reinterpret_cast<char*>(s_dyn4);
  char* s_lo = s_hi + NBP * HP;
  const int r = g.r;
  const int lane = wave_lane(), li = lane & 15, lg = lane >> 4;
  const int nwaves = gridDim.x * WPG;
  const int ntiles = (g.F + 15) / 16;
  const __amdgpu_buffer_rsrc_t qr = rsrc(g.Q, (uint32_t)((size_t)g.F * r * 2));
  const __amdgpu_buffer_rsrc_t cr = rsrc(g.c, (uint32_t)((size_t)g.F * 4));
  int tt = blockIdx.x * WPG + wave_id();
  uint4 q[NKB][4];
  float4 cv;
  // a tile's Q rows and the c of its result rows 4 lg + v, all requested at once (rows past F
  // read as zeros)
  auto load_tile = [&](int t) {
    const int i0 = t * 16 + 4 * lg;
    cv = __builtin_bit_cast(float4, bld16(cr, i0 < g.F ? (uint32_t)i0 * 4 : kNoRow));
    const int i = t * 16 + li;
    const uint32_t base = i < g.F ? (uint32_t)(((size_t)i * r + lg * 32) * 2) : kNoRow;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s = 0; s < 4; ++s) q[kb][s] = bld16(qr, base + kb * 256 + s * 16);
  };
  if (tt < ntiles) load_tile(tt);  // the first tile goes out before h is staged
  {
    constexpr int PER_ROW = NKB * 16;  // 16-byte pieces per padded token row
    constexpr int PIECES = 2 * NBP * PER_ROW;
    const __amdgpu_buffer_rsrc_t hr = rsrc(g.hhi, (uint32_t)(NBP * r * 2));
    const __amdgpu_buffer_rsrc_t lr = rsrc(g.hlo, (uint32_t)(NBP * r * 2));
    for (int p0 = threadIdx.x; p0 < PIECES; p0 += 4 * kBqFullThreads) {
      uint4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pc = p0 + k * kBqFullThreads;
        const int part = pc / (NBP * PER_ROW), rem = pc % (NBP * PER_ROW);
        const int n = rem / PER_ROW, e = (rem % PER_ROW) * 8;
        const uint32_t off = (pc < PIECES && e < r) ? (uint32_t)((n * r + e) * 2) : kNoRow;
        v[k] = bld16(part == 0 ? hr : lr, off);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pc = p0 + k * kBqFullThreads;
        if (pc < PIECES) {
          const int part = pc / (NBP * PER_ROW), rem = pc % (NBP * PER_ROW);
          const int n = rem / PER_ROW, e8 = rem % PER_ROW;
          *reinterpret_cast<uint4*>((part == 0 ? s_hi : s_lo) + n * HP + e8 * 16) = v[k];
        }
      }
    }
  }
  __syncthreads();
  for (; tt < ntiles; tt += nwaves) {
    f4_t acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = kb * 128 + lg * 32 + s * 8;
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const int o = (u * 16 + li) * HP + e * 2;
          const uint4 hh = *reinterpret_cast<const uint4*>(s_hi + o);
          const uint4 hl = *reinterpret_cast<const uint4*>(s_lo + o);
          acc[u] = mma(as_h8(q[kb][s]), as_h8(hh), acc[u]);
          acc[u] = mma(as_h8(q[kb][s]), as_h8(hl), acc[u]);
        }
        // keep the LDS reads of later steps from being hoisted (register pressure)
        if (s == 3) __builtin_amdgcn_sched_barrier(0);
      }
    const float cvv[4] = {cv.x, cv.y, cv.z, cv.w};
    uint32_t half = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = tt * 16 + 4 * lg + v;
      unsigned long long any = 0;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int n = u * 16 + li;
        const float l = acc[u][v] + cvv[v];
        const bool ok = n < g.B && i < g.F;
        if (g.logits && ok) g.logits[(size_t)n * g.F + i] = l;
        any |= __ballot(ok && l > g.thr);
      }
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        if ((any >> (16 * gg)) & 0xffffull) half |= 1u << (4 * gg + v);
    }
    if (lane == 0) reinterpret_cast<uint16_t*>(g.masks)[tt] = (uint16_t)half;
    if (tt + nwaves < ntiles) load_tile(tt + nwaves);
  }
}

// k_bscan: one workgroup orders the list: idx (ascending) and count from the mask words
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_bscan(BArgs g) {
  extern __shared__ uint32_t s_dyn[];
  uint32_t* s_mask = s_dyn;
  int* s_pre = reinterpret_cast<int*>(s_dyn + g.nq);
  __shared__ int s_red[kScanThreads / kWave];
  mask_prefix<kScanThreads>(g.masks, g.nq, g.n_hot, s_mask, s_pre, s_red);
  const int total = min(s_pre[g.nq], g.F);
  if (threadIdx.x == 0) *g.count_out = total;
  for (int q = threadIdx.x; q < g.nq; q += kScanThreads) {
    uint32_t m = s_mask[q];
    int at = s_pre[q];
    while (m) {
      const int b = __builtin_ctz(m);
      if (at < g.F) g.idx_out[at] = q * 32 + b;
      ++at;
      m &= m - 1u;
    }
  }
}

// =============================================================================================
// k_bup: unit (row block rb, chunk kc): list positions [64 rb, 64 rb + 64) (16 per wave) x
// d-elements [KC kc, KC kc + KC).  The chunk of x (all NBP token rows) is staged in LDS; the
// partial pre-activations go to upart/gpart[kc][n][k].  Grid-stride over the units.  Per unit the
// x chunk (L2) is requested first, then the weight rows (HBM), so that the LDS staging does not
// wait behind the weights.

template <St WT> struct BUp;
template <> struct BUp<St::F16> { static constexpr int LPB = 4; };  // 16-byte loads per lane per block
template <> struct BUp<St::I4> { static constexpr int LPB = 1; };

template <int KC>
__host__ __device__ constexpr int bup_xpitch() { return KC * 2 + 16; }
// bytes of LDS for the mask words and their prefix counts (scan mode of the up kernel)
__host__ __device__ inline size_t bup_scan_lds(int nq) { return ((size_t)8 * nq + 4 + 15) / 16 * 16; }

// SCAN (the layer call): the list is not given; every workgroup builds the prefix counts of the
// predictor's mask words in LDS (after the x chunk region) and each lane finds the neuron of its list
// position itself.  The chunk-0 units write the list and workgroup 0 its length, for the kernels
// that follow.
template <St WT, psffn_act ACT, int NT, int KC, bool SCAN>
__global__ __launch_bounds__(kBlock) void k_bup(BArgs g) {
  constexpr int NBP = 16 * NT;
  constexpr int KB = KC / 128;
  constexpr int LPB = BUp<WT>::LPB;
  constexpr int XP = bup_xpitch<KC>();
  constexpr bool GATE = ACT == PSFFN_SWIGLU;
  constexpr int PIECES = NBP * KC / 8;             // 16-byte pieces of the x chunk
  constexpr int PPT = (PIECES + kBlock - 1) / kBlock;  // per thread
  static_assert(KB <= 8, "scales of one unit row fit one 16-byte load");
  extern __shared__ uint4 s_dyn4[];
  char* s_x = reinterpret_cast<char*>(s_dyn4);
  const int lane = wave_lane(), li = lane & 15, lg = lane >> 4, wv = wave_id();
  const int d = g.d;
  int n_list;
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(s_x + NBP * XP);
  int* s_pre = reinterpret_cast<int*>(s_mask + g.nq);
  if constexpr (SCAN) {
    __shared__ int s_red[kBlock / kWave];
    mask_prefix<kBlock>(g.masks, g.nq, g.n_hot, s_mask, s_pre, s_red);
    n_list = min(s_pre[g.nq], g.F);
    if (blockIdx.x == 0 && threadIdx.x == 0) *g.count_out = n_list;
  } else {
    n_list = blist_len(g.count, g.F);
  }
  const int nrb = (n_list + 63) / 64;
  const int nkc = (d + KC - 1) / KC;
  const int units = nrb * nkc;
  const size_t rb_bytes = WT == St::I4 ? (size_t)d / 2 : (size_t)d * 2;
  const int ng = d / 128;  // 4-bit scale groups per row
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int kc = unit % nkc, rb = unit / nkc;  // consecutive units: consecutive chunks of the same rows
    // this lane's A row (list position) first, then the x chunk (rows n < NBP, elements
    // [KC kc, KC kc + KC), zero past B or d), then the weight rows once the neuron id is back
    const int k = rb * 64 + wv * 16 + li;
    int i_raw;
    if constexpr (SCAN) {
      i_raw = list_at(s_mask, s_pre, g.nq, k < n_list ? k : n_list - 1);
      if (kc == 0 && k < n_list && lg == 0) g.idx_out[k] = i_raw;
    } else {
      i_raw = g.idx[k < n_list ? k : n_list - 1];
    }
    uint4 xs[PPT];
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int pc = threadIdx.x + q * kBlock;
      const int n = pc / (KC / 8), e = kc * KC + (pc % (KC / 8)) * 8;
      xs[q] = ld16_or0(g.x + (size_t)n * d + e, pc < PIECES && n < g.B && e < d, g.x);
    }
    const bool valid = k < n_list && (unsigned)i_raw < (unsigned)g.F;
    const int i = valid ? i_raw : 0;
    const char* urow = reinterpret_cast<const char*>(g.w_up) + (size_t)i * rb_bytes;
    const char* grow = GATE ? reinterpret_cast<const char*>(g.w_gate) + (size_t)i * rb_bytes : nullptr;
    uint4 wu[KB][LPB], wg[KB][LPB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s = 0; s < LPB; ++s) {
        const int e = kc * KC + kb * 128 + lg * 32 + s * 8;
        const bool in = valid && e < d;
        const size_t off = WT == St::I4 ? (size_t)e / 2 : (size_t)e * 2;
        wu[kb][s] = ld16_or0(urow + off, in, g.w_up);
        if constexpr (GATE) wg[kb][s] = ld16_or0(grow + off, in, g.w_gate);
      }
    // 4-bit: this row's scales of the chunk's KB groups, packed in pairs, later handed to the
    // lanes holding the result rows; groups past the row's end stay zero (so do their weights)
    uint32_t su_w[4] = {0, 0, 0, 0}, sg_w[4] = {0, 0, 0, 0};
    if constexpr (WT == St::I4) {
      const int G0 = (kc * KC) / 128;
      const uint16_t* sp = g.s_up + (size_t)i * ng;
      const uint16_t* gp = GATE ? g.s_gate + (size_t)i * ng : nullptr;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int G = G0 + j;
        su_w[j / 2] |= ld16b_or0(sp + G, valid && G < ng, g.s_up) << (16 * (j & 1));
        if constexpr (GATE) sg_w[j / 2] |= ld16b_or0(gp + G, valid && G < ng, g.s_gate) << (16 * (j & 1));
      }
    }
    __syncthreads();  // the previous unit's reads of s_x are done
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int pc = threadIdx.x + q * kBlock;
      if (pc < PIECES) {
        const int n = pc / (KC / 8), el = (pc % (KC / 8)) * 8;
        *reinterpret_cast<uint4*>(s_x + n * XP + el * 2) = WT == St::I4 ? pair_x8(xs[q]) : xs[q];
      }
    }
    __syncthreads();
    float su[KB][4], sg[KB][4];
    if constexpr (WT == St::I4) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int w2 = 0; w2 < KB / 2; ++w2) {
          const uint32_t pu = (uint32_t)__shfl((int)su_w[w2], 4 * lg + v, kWave);
          su[2 * w2][v] = h2f(pu & 0xffffu);
          su[2 * w2 + 1][v] = h2f(pu >> 16);
          if constexpr (GATE) {
            const uint32_t pg = (uint32_t)__shfl((int)sg_w[w2], 4 * lg + v, kWave);
            sg[2 * w2][v] = h2f(pg & 0xffffu);
            sg[2 * w2 + 1][v] = h2f(pg >> 16);
          }
        }
    }
    f4_t au[NT], ag[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) au[t] = ag[t] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f4_t tu[NT], tg[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) tu[t] = tg[t] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int el = kb * 128 + lg * 32 + s * 8;
        h8_t fu, fg;
        if constexpr (WT == St::I4) {
          const uint32_t wdu = s == 0 ? wu[kb][0].x : s == 1 ? wu[kb][0].y : s == 2 ? wu[kb][0].z : wu[kb][0].w;
          fu = i4_frag(wdu);
          if constexpr (GATE) {
            const uint32_t wdg = s == 0 ? wg[kb][0].x : s == 1 ? wg[kb][0].y : s == 2 ? wg[kb][0].z : wg[kb][0].w;
            fg = i4_frag(wdg);
          }
        } else {
          fu = as_h8(wu[kb][s]);
          if constexpr (GATE) fg = as_h8(wg[kb][s]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const h8_t xf = as_h8(*reinterpret_cast<const uint4*>(s_x + (t * 16 + li) * XP + el * 2));
          if constexpr (WT == St::I4) {
            tu[t] = mma(fu, xf, tu[t]);
            if constexpr (GATE) tg[t] = mma(fg, xf, tg[t]);
          } else {
            au[t] = mma(fu, xf, au[t]);
            if constexpr (GATE) ag[t] = mma(fg, xf, ag[t]);
          }
        }
      }
      if constexpr (WT == St::I4) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            au[t][v] = fmaf(su[kb][v], tu[t][v], au[t][v]);
            if constexpr (GATE) ag[t][v] = fmaf(sg[kb][v], tg[t][v], ag[t][v]);
          }
      }
    }
    // partials: rows k0 .. k0+3 of token n, 16 bytes per lane
    const int k0 = rb * 64 + wv * 16 + 4 * lg;
    if (k0 < n_list) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const size_t o = ((size_t)kc * NBP + t * 16 + li) * g.ldk + k0;
        *reinterpret_cast<float4*>(g.upart + o) = make_float4(au[t][0], au[t][1], au[t][2], au[t][3]);
        if constexpr (GATE)
          *reinterpret_cast<float4*>(g.gpart + o) = make_float4(ag[t][0], ag[t][1], ag[t][2], ag[t][3]);
      }
    }
  }
}

// k_bact: a[n][k] for list positions k < roundup(count, 32) and tokens n < NBP (zero past the
// list and for padded tokens): the chunk partials summed in chunk order, plus bias, activation.
// Written as fp32 (4-bit down projection scales it per column group) and as fp16 hi/lo parts.
template <psffn_act ACT>
__global__ __launch_bounds__(kBlock) void k_bact(BArgs g, int nkc, int nbp) {
  const int n_list = blist_len(g.count, g.F);
  const int kpad = (n_list + 31) & ~31;
  const int total = nbp * kpad;
  for (int t = blockIdx.x * kBlock + threadIdx.x; t < total; t += gridDim.x * kBlock) {
    const int n = t / kpad, k = t % kpad;
    float a = 0.f;
    if (k < n_list && n < g.B) {
      // the neuron id (for its biases) and the chunk partials are requested together
      const int i = g.idx[k];
      constexpr int kR = 16;  // chunk partials in flight per round (one round up to 16 chunks)
      float su = 0.f, sg = 0.f;
      for (int c0 = 0; c0 < nkc; c0 += kR) {
        float pu[kR], pg[kR];
#pragma unroll
        for (int q = 0; q < kR; ++q) {
          const size_t o = ((size_t)(c0 + q) * nbp + n) * g.ldk + k;
          pu[q] = c0 + q < nkc ? g.upart[o] : 0.f;
          pg[q] = (ACT == PSFFN_SWIGLU && c0 + q < nkc) ? g.gpart[o] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < kR; ++q)
          if (c0 + q < nkc) {
            su += pu[q];
            if constexpr (ACT == PSFFN_SWIGLU) sg += pg[q];
          }
      }
      if ((unsigned)i < (unsigned)g.F) {
        su += g.b_up ? g.b_up[i] : 0.f;
        if constexpr (ACT == PSFFN_SWIGLU) {
          sg += g.b_gate ? g.b_gate[i] : 0.f;
          a = sg / (1.f + expf(-sg)) * su;
        } else {
          a = su > 0.f ? su : 0.f;
        }
      }
    }
    const size_t o = (size_t)n * g.ldk + k;
    g.aT[o] = a;
    _Float16 hi, lo;
    split_hl(a, hi, lo);
    g.ahi[o] = __builtin_bit_cast(uint16_t, hi);
    g.alo[o] = __builtin_bit_cast(uint16_t, lo);
  }
}

// =============================================================================================
// k_bdown: workgroup (column tile of 256, split s); wave w owns columns [col0, col0 + 64) and
// walks the split's list positions in steps of 32 rows.  The split's neuron ids are staged in LDS
// first; then a ring of D steps of loads (weight block, activation fragments, 4-bit scale) stays in
// flight per wave, refilled as each step is consumed.  Each step's 32 x 64 weight block goes
// through the wave's own LDS region (4-bit: decoded to fp16) and comes back transposed as A
// operands (columns x rows); the B operands are the activations of the 32 rows (hi and lo parts;
// 4-bit: times the rows' scales of this column group).  partial[s][n][col] for n < B.

template <St WT, int NT> struct BDn;
template <int NT> struct BDn<St::I4, NT> { static constexpr int LPS = 1; static constexpr int CS = NT == 1 ? 16 : 8; };
template <int NT> struct BDn<St::F16, NT> { static constexpr int LPS = 4; static constexpr int CS = 8; };

template <St WT, int NT>
__host__ __device__ constexpr int bdown_chunk_rows() { return BDn<WT, NT>::CS * 32; }
template <St WT, int NT>
__host__ __device__ constexpr int bdown_apitch() { return bdown_chunk_rows<WT, NT>() * 4 + 16; }
template <St WT, int NT>
__host__ __device__ constexpr size_t bdown_lds() {
  return (size_t)16 * NT * bdown_apitch<WT, NT>() + (size_t)bdown_chunk_rows<WT, NT>() * 4;
}

// XCD-contiguous column tiles: grid.x = 8 ceil(T / 8); workgroup x takes tile (x % 8) ceil(T / 8) + x / 8
// (a bijection of [0, grid.x); tiles >= T do nothing)
__host__ __device__ inline int bdown_grid_x(int T) { return 8 * ((T + 7) / 8); }
__host__ __device__ inline int bdown_tile(int x, int T) { return (x % 8) * ((T + 7) / 8) + x / 8; }

typedef short s4_t __attribute__((ext_vector_type(4)));
// gfx950 transposing LDS read of four 16-bit elements (one 8-byte piece named per lane)
__device__ __forceinline__ s4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)(p));
}

// 8 nibbles (columns c..c+7 of one row) -> 8 fp16 in column order: each byte pair of the
// flipped nibbles is placed under the fp16 exponent of 1024 (1024 + q + 8 exactly), then 1032 is
// subtracted from both halves
__device__ __forceinline__ void nib8_to_f16(uint32_t w, uint32_t (&o)[4]) {
  const uint32_t f = w ^ 0x88888888u;
  const uint32_t lo = f & 0x0F0F0F0Fu, hi = (f >> 4) & 0x0F0F0F0Fu;
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // bytes [lo.p, 0, hi.p, 0]: columns 2p (low half) and 2p + 1 (high half)
    const uint32_t sel = 0x0C000C00u | (uint32_t)p | ((uint32_t)(4 + p) << 16);
    const uint32_t v = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
    o[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v) - off);
  }
}

template <St WT, int NT>
__global__ __launch_bounds__(kBlock) void k_bdown(BArgs g) {
  constexpr int LPS = BDn<WT, NT>::LPS;
  constexpr int CS = BDn<WT, NT>::CS;
  constexpr int CR = CS * 32;
  constexpr int NBP = 16 * NT;
  constexpr int AP = bdown_apitch<WT, NT>();
  __shared__ __align__(16) char s_w[kBlock / kWave][32 * kDPitch];
  __shared__ __align__(16) float s_sc[kBlock / kWave][32];
  extern __shared__ uint4 s_dyn4[];
  char* s_a = reinterpret_cast<char*>(s_dyn4);             // activations of the chunk, per token row
  int* s_idx = reinterpret_cast<int*>(s_a + NBP * AP);      // neuron ids of the chunk
  const int lane = wave_lane(), li = lane & 15, lg = lane >> 4, wv = wave_id();
  const int d = g.d;
  const int n_list = blist_len(g.count, g.F);
  const int rowb = WT == St::I4 ? d / 2 + 2 * (d / 128) : 2 * d;
  int ks, S;
  bsplit(n_list, g.B, d, rowb, CR, ks, S);
  const int s = blockIdx.y;
  // column tile: 4-bit rows give each XCD (workgroups are dealt to the eight XCDs in turn) a
  // contiguous range of tiles, so that the few bytes of a row's group scales that neighbouring
  // tiles need come through one L2 instead of eight (cfg-3 shape at 8 tokens 103.4 -> 102.5 us);
  // fp16 rows keep tile = blockIdx.x
  const int T = (d + 255) / 256;
  const int tile = WT == St::I4 ? bdown_tile(blockIdx.x, T) : (int)blockIdx.x;
  if (s >= S || tile >= T) return;
  const int col0 = tile * 256 + wv * 64;
  const int k_lo = s * ks;
  const int nrows = min(n_list, k_lo + ks) - k_lo;
  const int srow = lane >> 1, shalf = lane & 1;  // staging: row of the step, 32-column half
  char* wbuf = s_w[wv];
  const uint32_t row_stride = WT == St::I4 ? (uint32_t)d / 2 : (uint32_t)d * 2;
  const int ng = d / 128;
  const __amdgpu_buffer_rsrc_t wr_rs = rsrc(g.w_dT, (uint32_t)((size_t)g.F * row_stride));
  const __amdgpu_buffer_rsrc_t sc_rs = rsrc(g.s_dT, WT == St::I4 ? (uint32_t)((size_t)g.F * ng * 2) : 0u);
  f4_t acc[4][NT];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nrows; c0 += CR) {
    const int crows = min(CR, nrows - c0);
    const int csteps = (crows + 31) / 32;
    if (c0 > 0) __syncthreads();  // the previous chunk's LDS reads are done
    // the chunk's neuron ids and activations (rows < csteps * 32 <= roundup(count, 32): the
    // activations there are zero-filled), requested together
    {
      constexpr int PR = WT == St::I4 ? CR / 4 : CR / 8;  // 16-byte pieces per token row (per part)
      constexpr int PARTS = WT == St::I4 ? 1 : 2;
      constexpr int PIECES = NBP * PR * PARTS;
      constexpr int PPT = (PIECES + kBlock - 1) / kBlock;
      const int live_pr = WT == St::I4 ? csteps * 8 : csteps * 4;
      int iv[(CR + kBlock - 1) / kBlock];
#pragma unroll
      for (int q = 0; q < (CR + kBlock - 1) / kBlock; ++q) {
        const int j = threadIdx.x + q * kBlock;
        iv[q] = j < crows ? g.idx[k_lo + c0 + j] : -1;
      }
      uint4 av[PPT];
#pragma unroll
      for (int q = 0; q < PPT; ++q) {
        const int pc = threadIdx.x + q * kBlock;
        const int part = pc / (NBP * PR), rem = pc % (NBP * PR);
        const int n = rem / PR, e = rem % PR;
        const bool ok = pc < PIECES && e < live_pr;
        const size_t kk = (size_t)k_lo + c0 + (size_t)e * (WT == St::I4 ? 4 : 8);
        const void* src = WT == St::I4 ? static_cast<const void*>(g.aT + (size_t)n * g.ldk + kk)
                                       : static_cast<const void*>((part == 0 ? g.ahi : g.alo) + (size_t)n * g.ldk + kk);
        av[q] = ld16_or0(src, ok, nullptr);
      }
#pragma unroll
      for (int q = 0; q < (CR + kBlock - 1) / kBlock; ++q) {
        const int j = threadIdx.x + q * kBlock;
        if (j < CR) s_idx[j] = (unsigned)iv[q] < (unsigned)g.F ? iv[q] : -1;
      }
#pragma unroll
      for (int q = 0; q < PPT; ++q) {
        const int pc = threadIdx.x + q * kBlock;
        if (pc < PIECES) {
          const int part = pc / (NBP * PR), rem = pc % (NBP * PR);
          const int n = rem / PR, e = rem % PR;
          *reinterpret_cast<uint4*>(s_a + n * AP + part * (CR * 2) + e * 16) = av[q];
        }
      }
    }
    __syncthreads();
    // every weight slice of the chunk in flight at once (rows past the list read zeros)
    uint4 wr[CS][LPS];
    uint32_t scb[CS];
#pragma unroll
    for (int st = 0; st < CS; ++st) {
      const int rr = st * 32 + srow;
      const int i = (st < csteps && rr < crows) ? s_idx[rr] : -1;
      const uint32_t rbase = i >= 0 ? (uint32_t)i * row_stride : kNoRow;
#pragma unroll
      for (int q = 0; q < LPS; ++q) {
        const int c = col0 + shalf * 32 + q * 8;
        const uint32_t cb = WT == St::I4 ? (uint32_t)c / 2 : (uint32_t)c * 2;
        wr[st][q] = bld16(wr_rs, c < d ? rbase + cb : kNoRow);  // kNoRow + cb stays out of range
      }
      if constexpr (WT == St::I4) {
        const int G = col0 / 128;
        scb[st] = __builtin_amdgcn_raw_buffer_load_b16(sc_rs, (i >= 0 && G < ng) ? ((uint32_t)i * ng + G) * 2 : kNoRow,
                                                       0, 0);
      }
    }
#pragma unroll
    for (int st = 0; st < CS; ++st) {
      if (st < csteps) {  // (no break: the loop must unroll so that wr[st] stays in registers)
      // stage the 32 x 64 block: row srow, columns [32 shalf, 32 shalf + 32), as fp16
      char* dst = wbuf + srow * kDPitch + shalf * 64;
      if constexpr (WT == St::I4) {
        const uint32_t wd[4] = {wr[st][0].x, wr[st][0].y, wr[st][0].z, wr[st][0].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t o4[4];
          nib8_to_f16(wd[q], o4);
          *reinterpret_cast<uint2*>(dst + q * 16) = make_uint2(o4[0], o4[1]);
          *reinterpret_cast<uint2*>(dst + q * 16 + 8) = make_uint2(o4[2], o4[3]);
        }
        if (shalf == 0) s_sc[wv][srow] = h2f(scb[st]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<uint2*>(dst + q * 16) = make_uint2(wr[st][q].x, wr[st][q].y);
          *reinterpret_cast<uint2*>(dst + q * 16 + 8) = make_uint2(wr[st][q].z, wr[st][q].w);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // B operands: rows 8 lg .. 8 lg + 8 of the step, token li (+16 t)
      h8_t fb_hi[NT], fb_lo[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const char* arow = s_a + (t * 16 + li) * AP;
        if constexpr (WT == St::I4) {
          const float4 a0 = *reinterpret_cast<const float4*>(arow + (st * 32 + lg * 8) * 4);
          const float4 a1 = *reinterpret_cast<const float4*>(arow + (st * 32 + lg * 8) * 4 + 16);
          const float4 s0 = *reinterpret_cast<const float4*>(&s_sc[wv][lg * 8]);
          const float4 s1 = *reinterpret_cast<const float4*>(&s_sc[wv][lg * 8 + 4]);
          const float pv[8] = {a0.x * s0.x, a0.y * s0.y, a0.z * s0.z, a0.w * s0.w,
                               a1.x * s1.x, a1.y * s1.y, a1.z * s1.z, a1.w * s1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            _Float16 hi, lo;
            split_hl(pv[j], hi, lo);
            fb_hi[t][j] = hi;
            fb_lo[t][j] = lo;
          }
        } else {
          fb_hi[t] = as_h8(*reinterpret_cast<const uint4*>(arow + (st * 32 + lg * 8) * 2));
          fb_lo[t] = as_h8(*reinterpret_cast<const uint4*>(arow + CR * 2 + (st * 32 + lg * 8) * 2));
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // A operand (column 16 m + li, rows 8 lg .. 8 lg + 8) by two transposing LDS reads: within
        // a group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces named by lanes
        // i / 4 + 4 j (j < 4), so lane 4 j + a names row 8 lg + 4 h + j, columns 16 m + 4 a .. + 4
        const char* src = wbuf + (lg * 8 + (li >> 2)) * kDPitch + (m * 16 + (li & 3) * 4) * 2;
        const s4_t r0 = lds_read_tr16(src), r1 = lds_read_tr16(src + 4 * kDPitch);
        // (joined as one vector: element-wise extraction of these results miscompiles)
        const h8_t fa = __builtin_bit_cast(h8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[m][t] = mma(fa, fb_hi[t], acc[m][t]);
          acc[m][t] = mma(fa, fb_lo[t], acc[m][t]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      }
    }
  }
  // D[col 16 m + 4 lg + v][token li + 16 t]
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int c = col0 + m * 16 + 4 * lg;
    if (c >= d) continue;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = t * 16 + li;
      if (n < g.B)
        *reinterpret_cast<float4*>(g.part + ((size_t)s * g.B + n) * d + c) =
            make_float4(acc[m][t][0], acc[m][t][1], acc[m][t][2], acc[m][t][3]);
    }
  }
}

// k_breduce: y[n][j] = (accumulate ? y : 0) + (b_down[j] + sum over splits in split order)
__global__ __launch_bounds__(kBlock) void k_breduce(BArgs g, int rowb, int chunk_rows) {
  const int n_list = blist_len(g.count, g.F);
  int ks, S;
  bsplit(n_list, g.B, g.d, rowb, chunk_rows, ks, S);
  const size_t t = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (size_t)g.B * g.d) return;
  const int col = (int)(t % g.d);
  float v = g.b_down ? g.b_down[col] : 0.f;
  for (int s0 = 0; s0 < S; s0 += 16) {
    float pv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) pv[u] = s0 + u < S ? g.part[(size_t)(s0 + u) * g.B * g.d + t] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (s0 + u < S) v += pv[u];
  }
  g.y[t] = g.accumulate ? g.y[t] + v : v;
}

// =============================================================================================
// host side

// scratch layout of the batch pipeline (offsets from the workspace scratch start); the predictor
// and the FFN regions overlap: a layer runs them in stream order
struct BLayout {
  size_t hpart, hhi, hlo, pred_end;
  size_t upart, gpart, aT, ahi, alo, part, ffn_end;
};

static int nbp_of(int B) { return B <= 16 ? 16 : 32; }
static int up_kc(St wt, int nbp) { return (wt == St::I4 && nbp == 16) ? 1024 : 512; }

static BLayout blayout(int B, int d, int r, int F, St wt, bool gate) {
  BLayout L{};
  const int nbp = nbp_of(B);
  const size_t ksh = (size_t)(d + kHChunk - 1) / kHChunk;
  L.hpart = 0;
  L.hhi = round256(ksh * nbp * r * 4);
  L.hlo = L.hhi + round256((size_t)nbp * r * 2);
  L.pred_end = L.hlo + round256((size_t)nbp * r * 2);
  const size_t ldk = (size_t)((F + 31) & ~31);
  const size_t nkc = (size_t)(d + up_kc(wt, nbp) - 1) / up_kc(wt, nbp);
  L.upart = 0;
  L.gpart = round256(nkc * nbp * ldk * 4);
  L.aT = L.gpart + (gate ? L.gpart : 0);
  L.ahi = L.aT + round256((size_t)nbp * ldk * 4);
  L.alo = L.ahi + round256((size_t)nbp * ldk * 2);
  L.part = L.alo + round256((size_t)nbp * ldk * 2);
  L.ffn_end = L.part + round256((size_t)kBSplitCap * B * (size_t)d * 4);
  return L;
}

size_t batch_scratch_bytes(int B, int d, int r, int F, psffn_dtype wdt, psffn_act act, bool pred, bool ffn) {
  const St wt = wdt == PSFFN_I4G128 ? St::I4 : St::F16;
  const BLayout L = blayout(B, d, r > 0 ? r : 8, F, wt, act == PSFFN_SWIGLU);
  size_t need = 0;
  if (pred) need = L.pred_end;
  if (ffn && L.ffn_end > need) need = L.ffn_end;
  return need;
}

bool batch_supported_pred(const psffn_predictor& P, int B) {
  return B >= 2 && B <= 32 && P.dt == PSFFN_F16 && P.F <= kBatchMaxF &&
         (size_t)P.r * P.d * 2 <= kMaxBufferBytes;  // k_bh reads A through one buffer resource
}
bool batch_supported_ffn(const psffn_ffn& W, int B) {
  const size_t rowb = W.dt == PSFFN_I4G128 ? (size_t)W.d / 2 : (size_t)W.d * 2;
  return B >= 2 && B <= 32 && (W.dt == PSFFN_F16 || W.dt == PSFFN_I4G128) && W.F <= kBatchMaxF &&
         (size_t)W.F * rowb <= kMaxBufferBytes;
}

static void pred_args(BArgs& g, const psffn_predictor& P, const void* x, int B, float thr, float* logits, void* ws) {
  const StateLayout S = state_layout(P.F);
  char* w = static_cast<char*>(ws);
  const BLayout L = blayout(B, P.d, P.r, P.F, St::F16, false);
  char* sc = w + S.scratch;
  g.A = static_cast<const uint16_t*>(P.A);
  g.Q = static_cast<const uint16_t*>(P.Q);
  g.c = P.c;
  g.r = P.r;
  g.thr = thr;
  g.logits = logits;
  g.hpart = reinterpret_cast<float*>(sc + L.hpart);
  g.hhi = reinterpret_cast<uint16_t*>(sc + L.hhi);
  g.hlo = reinterpret_cast<uint16_t*>(sc + L.hlo);
  g.masks = reinterpret_cast<uint32_t*>(w + S.masks);
  g.nq = (P.F + 31) / 32;
  g.x = static_cast<const uint16_t*>(x);
  g.B = B;
  g.d = P.d;
  g.F = P.F;
}

static void ffn_args_b(BArgs& g, const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count,
                       float* y, int accumulate, void* ws) {
  const StateLayout S = state_layout(W.F);
  char* w = static_cast<char*>(ws);
  const St wt = W.dt == PSFFN_I4G128 ? St::I4 : St::F16;
  const BLayout L = blayout(B, W.d, 8, W.F, wt, W.act == PSFFN_SWIGLU);
  char* sc = w + S.scratch;
  g.x = static_cast<const uint16_t*>(x);
  g.B = B;
  g.d = W.d;
  g.F = W.F;
  g.w_up = W.w_up;
  g.w_gate = W.w_gate;
  g.w_dT = W.w_dT;
  g.s_up = static_cast<const uint16_t*>(W.s_up);
  g.s_gate = static_cast<const uint16_t*>(W.s_gate);
  g.s_dT = static_cast<const uint16_t*>(W.s_dT);
  g.b_up = W.b_up;
  g.b_gate = W.b_gate;
  g.b_down = W.b_down;
  g.idx = idx;
  g.count = count;
  g.ldk = (W.F + 31) & ~31;
  g.upart = reinterpret_cast<float*>(sc + L.upart);
  g.gpart = reinterpret_cast<float*>(sc + L.gpart);
  g.aT = reinterpret_cast<float*>(sc + L.aT);
  g.ahi = reinterpret_cast<uint16_t*>(sc + L.ahi);
  g.alo = reinterpret_cast<uint16_t*>(sc + L.alo);
  g.part = reinterpret_cast<float*>(sc + L.part);
  g.y = y;
  g.accumulate = accumulate;
  g.masks = reinterpret_cast<uint32_t*>(w + S.masks);
  g.nq = (W.F + 31) / 32;
}

// LDS of the persistent logits kernel, 0 when h does not fit (then the kernel with h fragments
// read from L2 runs instead)
static size_t bq_lds(int nbp, int r) {
  const size_t b = 2 * (size_t)nbp * bq_pitch(r);
  return b <= (size_t)160 * 1024 ? b : 0;
}

template <int NT>
static hipError_t bq_lds_attr() {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bq_lds<NT>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  return e;
}

template <int NT, int NKB>
static hipError_t bq_full_attr() {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bq_full<NT, NKB>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  return e;
}

static int cu_count() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return v > 0 ? v : 256;
  }();
  return n;
}

template <int NT>
static hipError_t pred_launch(const BArgs& g, hipStream_t s) {
  const int nbp = 16 * NT;
  const int ksh = (g.d + kHChunk - 1) / kHChunk;
  k_bh<NT><<<dim3(ksh, (g.r + 63) / 64), kBlock, 0, s>>>(g);
  k_bhred<<<(nbp * g.r + kBlock - 1) / kBlock, kBlock, 0, s>>>(g, ksh, nbp);
  const size_t lds = bq_lds(nbp, g.r);
  const int nkb = (g.r + 127) / 128;
  const int nkb_t = nkb <= 4 ? 4 : (nkb <= 8 ? 8 : 12);
  const size_t lds_full = 2 * (size_t)nbp * bq_full_pitch(nkb_t);
  if (nkb <= 12 && lds_full <= (size_t)160 * 1024 && (size_t)g.F * g.r * 2 <= kMaxBufferBytes) {
    constexpr int kBqFullThreads = bq_full_threads<NT>();
    const int tiles = (g.F + 15) / 16, per_wg = kBqFullThreads / kWave;
    int grid = cu_count();
    if (grid > (tiles + per_wg - 1) / per_wg) grid = (tiles + per_wg - 1) / per_wg;
    hipError_t e;
    if (nkb <= 4) {
      e = bq_full_attr<NT, 4>();
      if (e == hipSuccess) k_bq_full<NT, 4><<<grid, kBqFullThreads, lds_full, s>>>(g);
    } else if (nkb <= 8) {
      e = bq_full_attr<NT, 8>();
      if (e == hipSuccess) k_bq_full<NT, 8><<<grid, kBqFullThreads, lds_full, s>>>(g);
    } else {
      e = bq_full_attr<NT, 12>();
      if (e == hipSuccess) k_bq_full<NT, 12><<<grid, kBqFullThreads, lds_full, s>>>(g);
    }
    if (e != hipSuccess) return e;
  } else if (lds) {
    const hipError_t e = bq_lds_attr<NT>();
    if (e != hipSuccess) return e;
    const int units = (g.F + 31) / 32, per_wg = kBqThreads / kWave;
    int grid = cu_count();
    if (grid > (units + per_wg - 1) / per_wg) grid = (units + per_wg - 1) / per_wg;
    k_bq_lds<NT><<<grid, kBqThreads, lds, s>>>(g);
  } else {
    k_bq<NT><<<(g.F + 127) / 128, kBlock, 0, s>>>(g);
  }
  return hipSuccess;
}

template <St WT, psffn_act ACT, int NT>
static void ffn_launch_b(const BArgs& g, hipStream_t s, bool scan) {
  constexpr int NBP = 16 * NT;
  constexpr int KC = (WT == St::I4 && NT == 1) ? 1024 : 512;
  const int nkc = (g.d + KC - 1) / KC;
  const size_t lds = (size_t)NBP * bup_xpitch<KC>();
  int units = ((g.F + 63) / 64) * nkc;
  if (units > 1024) units = 1024;
  if (scan)
    k_bup<WT, ACT, NT, KC, true><<<units, kBlock, lds + bup_scan_lds(g.nq), s>>>(g);
  else
    k_bup<WT, ACT, NT, KC, false><<<units, kBlock, lds, s>>>(g);
  int act_grid = (NBP * g.ldk + kBlock - 1) / kBlock;
  if (act_grid > 1024) act_grid = 1024;
  k_bact<ACT><<<act_grid, kBlock, 0, s>>>(g, nkc, NBP);
  const int rowb = WT == St::I4 ? g.d / 2 + 2 * (g.d / 128) : 2 * g.d;
  static_assert(bdown_lds<WT, NT>() + sizeof(char) * 4 * 32 * kDPitch + 4 * 32 * 4 <= 65536,
                "the down kernel stays within the default 64 KB of LDS");
  const int T = (g.d + 255) / 256;
  k_bdown<WT, NT><<<dim3(WT == St::I4 ? bdown_grid_x(T) : T, kBSplitCap), kBlock, bdown_lds<WT, NT>(), s>>>(g);
  k_breduce<<<(unsigned)(((size_t)g.B * g.d + kBlock - 1) / kBlock), kBlock, 0, s>>>(g, rowb,
                                                                                       bdown_chunk_rows<WT, NT>());
}

template <St WT, psffn_act ACT>
static void ffn_launch_nt(const BArgs& g, hipStream_t s, bool scan) {
  if (g.B <= 16) ffn_launch_b<WT, ACT, 1>(g, s, scan);
  else ffn_launch_b<WT, ACT, 2>(g, s, scan);
}

// The layer call lets the up kernel order the list for fp16 weights (measured on MI355X, one machine:
// OPT-30B shape at 4 tokens 60.3 -> 55.4 us, 48-layer stack at 4 and 32 tokens +2.5% and +1.4%
// tokens/s); for 4-bit weights the larger LDS footprint of their 1024-element x chunk costs more
// than the list kernel (OPT-175B shape at 8 tokens 107.2 -> 108.4 us), so they keep it.  The LDS
// (x chunk plus the mask words and their prefix counts) must fit the default 64 KB.
static bool bup_scan_fits(const psffn_ffn& W, int B, int nq) {
  if (W.dt != PSFFN_F16) return false;
  const int NT = B <= 16 ? 1 : 2;
  const int KC = (W.dt == PSFFN_I4G128 && NT == 1) ? 1024 : 512;
  return (size_t)16 * NT * (KC * 2 + 16) + bup_scan_lds(nq) <= (size_t)64 * 1024;
}

static void ffn_dispatch(const psffn_ffn& W, const BArgs& g, hipStream_t s, bool scan = false) {
  if (W.dt == PSFFN_I4G128) {
    if (W.act == PSFFN_RELU) ffn_launch_nt<St::I4, PSFFN_RELU>(g, s, scan);
    else ffn_launch_nt<St::I4, PSFFN_SWIGLU>(g, s, scan);
  } else {
    if (W.act == PSFFN_RELU) ffn_launch_nt<St::F16, PSFFN_RELU>(g, s, scan);
    else ffn_launch_nt<St::F16, PSFFN_SWIGLU>(g, s, scan);
  }
}

static hipError_t predict_and_scan(const BArgs& g, hipStream_t s) {
  const hipError_t e = g.B <= 16 ? pred_launch<1>(g, s) : pred_launch<2>(g, s);
  if (e != hipSuccess) return e;
  k_bscan<<<1, kScanThreads, 8 * (size_t)g.nq + 4, s>>>(g);
  return hipSuccess;
}

hipError_t launch_predict_batch_masks(const psffn_predictor& P, const void* x, int B, float thr, float* logits,
                                      void* ws, hipStream_t s) {
  if (!batch_supported_pred(P, B)) return hipErrorNotSupported;
  BArgs g{};
  pred_args(g, P, x, B, thr, logits, ws);
  const hipError_t e = g.B <= 16 ? pred_launch<1>(g, s) : pred_launch<2>(g, s);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_predict_batch(const psffn_predictor& P, const void* x, int B, float thr, int32_t* idx,
                                int32_t* count, float* logits, void* ws, hipStream_t s, int n_hot) {
  if (!batch_supported_pred(P, B)) return hipErrorNotSupported;
  BArgs g{};
  pred_args(g, P, x, B, thr, logits, ws);
  g.n_hot = n_hot;
  g.idx_out = idx;
  g.count_out = count;
  const hipError_t e = predict_and_scan(g, s);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_ffn_batch(const psffn_ffn& W, const void* x, int B, const int32_t* idx, const int32_t* count,
                            float* y, int accumulate, void* ws, hipStream_t s) {
  if (!batch_supported_ffn(W, B)) return hipErrorNotSupported;
  BArgs g{};
  ffn_args_b(g, W, x, B, idx, count, y, accumulate, ws);
  ffn_dispatch(W, g, s);
  return hipGetLastError();
}

hipError_t launch_layer_batch(const psffn_predictor& P, const psffn_ffn& W, const void* x, int B, float thr,
                              int32_t* idx, int32_t* count, float* logits, float* y, int accumulate, void* ws,
                              hipStream_t s, int n_hot) {
  if (!batch_supported_pred(P, B) || !batch_supported_ffn(W, B)) return hipErrorNotSupported;
  BArgs g{};
  pred_args(g, P, x, B, thr, logits, ws);
  g.n_hot = n_hot;
  g.idx_out = idx;
  g.count_out = count;
  BArgs f{};
  ffn_args_b(f, W, x, B, idx, count, y, accumulate, ws);
  if (bup_scan_fits(W, B, g.nq)) {
    // the up kernel orders the list from the mask words itself (no list kernel, one launch fewer)
    const hipError_t e = g.B <= 16 ? pred_launch<1>(g, s) : pred_launch<2>(g, s);
    if (e != hipSuccess) return e;
    f.masks = g.masks;
    f.nq = g.nq;
    f.n_hot = n_hot;
    f.idx_out = idx;
    f.count_out = count;
    ffn_dispatch(W, f, s, true);
    return hipGetLastError();
  }
  hipError_t e = predict_and_scan(g, s);
  if (e != hipSuccess) return e;
  ffn_dispatch(W, f, s);
  return hipGetLastError();
}

}  // namespace psffn

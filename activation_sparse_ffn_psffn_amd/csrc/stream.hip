// Streamed one-token pipeline for fp16 predictors and fp16 or 4-bit (g128) ReLU weights.
//
// Layer call, three kernels:
//   k_h1   h = A x, one single-wave workgroup per row of A (the bits of the small-batch k_h, which
//          takes over for rows longer than 12288 and for the stack step's LayerNorm)
//   k_qu   per chunk of 16 neurons: l = Q h + c, the threshold test and the chunk's mask bits, and
//          then, in the same workgroup, the up rows of the chunk's kept neurons,
//          a_i = max(W_up[i] . x + b_up[i], 0).  The up rows stream while other workgroups still
//          stream Q, instead of after the whole predictor.
//   k_dn   the down projection, y = b_down + sum_i a_i W_dT[i], by (column tile, split): split s
//          takes the kept neurons i with i mod S == s (in a hot-first layer the hot neurons are
//          low-indexed, so this spreads them evenly), column tile t takes 512 output columns (1 KB
//          of every fp16 row, 256 bytes of every 4-bit row).  Each workgroup writes its tile's
//          partial sum; the last of a tile's S workgroups to finish (a completion count per tile,
//          no spin-wait) adds the S partials in split order and writes y.  One more workgroup
//          writes the ascending list of kept neurons and its length.
// FFN call on a given list: k_up1 / k_up1_i4 (the up rows of the listed neurons, two at a time by
// a whole workgroup, the same arithmetic as k_qu) and k_dn in list mode (split s takes the list
// entries with i mod S == s, in list order).  On the ascending list of a predictor call that is the
// same sequence as the layer call's, so psffn_layer equals psffn_predict followed by
// psffn_sparse_ffn bit for bit.
//
// Method ("PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU", Elamur
// Research summary): Summary 2nd paragraph (a per-layer predictor guesses the firing neurons;
// neuron-level kernels compute those and skip the rest), Interesting ideas I4 (work on whole rows
// and columns of the weights, no sparse format) and I1 (hot parts first).
//
// Cross-workgroup data inside k_dn: the partials are written with device-scope (sc1) stores and
// read back with device-scope loads, so they are coherent across the XCDs' L2 caches without a
// cache write-back; every thread waits for its stores to complete before the workgroup takes its
// completion ticket.  The tickets are zeroed by the kernel before k_dn in the same call.
#include "chunk.h"
#include "common.h"

namespace psffn {

namespace {

constexpr int kTile = 512;      // output columns per k_dn workgroup (1 KB of an fp16 row, 16 B per lane)
constexpr int kSeg = 8;         // ids per thread per segment of k_dn's id gathering
constexpr int kDnRB = 8;        // rows per wave in flight in k_dn
constexpr int kCPL4 = 8;        // output columns per lane of the 4-bit k_dn (kCPL4 / 2 bytes of a row)
constexpr int kTile4 = kWave * kCPL4;  // output columns per 4-bit k_dn workgroup
constexpr int kDn4RB = 8;       // 4-bit rows per wave in flight in k_dn
constexpr int kUQ4 = 2;         // 32-element slices per lane per 4-bit up row: rows of up to 16384 elements
constexpr int kMaxWords = 8192;  // mask words the layer call takes (F <= 262144)
constexpr int kSW = 1;         // k_dn splits: 32 kSW (split s: neurons i with i mod 32 kSW == s)
constexpr int kMaxSplits = 32 * kSW;

__device__ uint4 s_zero16[1] = {{0u, 0u, 0u, 0u}};  // never written
__device__ float s_zero_f[1] = {0.f};               // never written

// Weight rows (rows of A, the kept neurons' up and down rows; Q in chunk.h) are read once per call.
// Their loads carry the non-temporal cache policy, so that the stream does not push out of L2 the
// lines that are read again: x, h, the mask words, the activations, the split partials and the
// kernels' code.  Each of these loads takes whole 128-byte lines in one instruction.  Measured on
// MI355X (same machine, alternating): OPT-30B-shaped layer at one token 31.5 -> 31.1 us,
// OPT-175B-shaped 4-bit layer 55.2 -> 53.2 us, 48-layer stack at one token +3.7% tokens/s.
constexpr int kNT = 2;  // the nt bit of a buffer load's cache-policy operand

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldz16_nt(const void* p, bool ok) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                       reinterpret_cast<const u32x4v*>(ok ? p : static_cast<const void*>(s_zero16))));
}

__device__ __forceinline__ void st_dev64(void* p, float lo, float hi) {
  const uint64_t v = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// exclusive prefix of v over the workgroup (kBlock threads) and the total; s_red holds the wave
// totals; ends with every thread past the barrier (s_red may be reused after the next barrier)
__device__ __forceinline__ int block_excl(int v, int* s_red, int& total) {
  const int lane = wave_lane(), wv = wave_id();
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == kWave - 1) s_red[wv] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    if (w < wv) off += s_red[w];
    tot += s_red[w];
  }
  total = tot;
  return off + inc - v;
}

// position (0-based) of the j-th set bit of m (j < popcount(m))
__device__ __forceinline__ int nth_bit(uint32_t m, int j) {
  for (int k = 0; k < j; ++k) m &= m - 1u;
  return __builtin_ctz(m);
}

// ---- one up row per wave: UN 16-byte slices (8 fp16) per lane per pass, x (fp16) in LDS

// Buffer loads (MUBUF): the resource holds a row's base address and byte size, the lane gives a
// 32-bit byte offset, and a read past the size returns zeros.  A whole row then takes one VGPR of
// offset (the per-slice steps are constants) and no predicate; a row of size 0 reads as zeros.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// resource of row i (wave-uniform; i < 0: an empty resource) of rows of row_bytes (< 2 GiB)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int i, uint32_t row_bytes) {
  const char* p = static_cast<const char*>(base) + (size_t)(i >= 0 ? i : 0) * row_bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, i >= 0 ? (int)row_bytes : 0, kRsrcWord3);
}

// Up rows by a whole workgroup, kRPG rows at a time.  Wave w covers the quarter [w S4, w S4 + S4)
// of a row's 16-byte slices (S4 = ceil(d / 32)); lane L takes slices w S4 + L + 64 u (u < kUQ), so
// rows of up to kUQ * 2048 fp16 elements.  The lane's x slices are loaded once.  A row's value is
// ((p0 + p1) + p2) + p3 over the four wave sums (each: the lane's slices in order, then the xor
// butterfly), the same whichever rows share the group.
constexpr int kUQ = 4;
constexpr int kRPG = 2;
constexpr int kIlv = 256;  // k_qu: chunks per interleave block (measured: 128 32.3, 256 32.0, 512 32.7,
                           // the whole range 33.2, contiguous chunks 41.2 us on the OPT-30B-shaped layer)
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every row: reads zeros

struct UpSlices {
  uint32_t off[kUQ];  // byte offsets of the lane's slices within a row (kOob: none)
};

__device__ __forceinline__ UpSlices up_slices(int d) {
  const int nsl = d / 8, S4 = (nsl + 3) / 4;
  const int w = wave_id(), L = wave_lane();
  UpSlices o;
#pragma unroll
  for (int u = 0; u < kUQ; ++u) {
    const int k = L + kWave * u, sl = w * S4 + k;
    o.off[u] = (k < S4 && sl < nsl) ? (uint32_t)sl * 16 : kOob;
  }
  return o;
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT));
}

__device__ __forceinline__ void x_slices(const _Float16* __restrict__ x, int d, const UpSlices& o, uint4 (&xv)[kUQ]) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(x), 0, d * 2, kRsrcWord3);
#pragma unroll
  for (int u = 0; u < kUQ; ++u) xv[u] = bload16(rs, o.off[u]);
}

// the lane's slices of rows ids[0..kRPG) (id < 0: zeros)
__device__ __forceinline__ void up_rows_load(const _Float16* __restrict__ w_up, int d, const int (&ids)[kRPG],
                                             const UpSlices& o, uint4 (&w)[kRPG][kUQ]) {
#pragma unroll
  for (int r = 0; r < kRPG; ++r) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(w_up, ids[r], (uint32_t)d * 2);
#pragma unroll
    for (int u = 0; u < kUQ; ++u) w[r][u] = bload16_nt(rs, o.off[u]);
  }
}

// a_i = max(W_up[i] . x + b_up[i], 0) for the group's rows; thread r (< kRPG) stores row r's value.
// s_p holds kRPG x 4 wave sums; two barriers (every thread of the workgroup calls it).
__device__ __forceinline__ void up_rows_finish(const uint4 (&w)[kRPG][kUQ], const uint4 (&xv)[kUQ],
                                               const int (&ids)[kRPG], const float* __restrict__ b_up,
                                               float* __restrict__ a, float* s_p) {
  const int lane = wave_lane(), wv = wave_id();
#pragma unroll
  for (int r = 0; r < kRPG; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kUQ; ++u) acc = dot8_f16(w[r][u], xv[u], acc);
    acc = wave_sum(acc);
    if (lane == 0) s_p[r * 4 + wv] = acc;
  }
  __syncthreads();
  if (threadIdx.x < kRPG) {
    const int r = threadIdx.x;
    int i = -1;
#pragma unroll
    for (int k = 0; k < kRPG; ++k)
      if (k == r) i = ids[k];
    if (i >= 0) {
      const float z = ((s_p[r * 4] + s_p[r * 4 + 1]) + s_p[r * 4 + 2]) + s_p[r * 4 + 3];
      const float v = z + (b_up ? b_up[i] : 0.f);
      a[i] = v > 0.f ? v : 0.f;
    }
  }
  __syncthreads();
}

// completion tickets, one per 256-byte line (atomics on one line serialise)
constexpr int kTicketStride = 64;  // 32-bit words

__device__ __forceinline__ void zero_tickets(uint32_t* ctr, int T) {
  for (int k = threadIdx.x; k < T; k += kBlock)
    __hip_atomic_store(ctr + k * kTicketStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// =========================================================================================
// k_up1: a_i for the neurons of a given list (FFN call), kRPG list entries per workgroup at a time;
// entries outside [0, F) are skipped.  Workgroup 0 also zeroes k_dn's completion tickets.

struct UpArgs {
  const int32_t* idx;
  const int32_t* count;
  const _Float16* w_up;
  const float* b_up;
  const _Float16* x;
  float* a;
  uint32_t* ctr;
  int F, d, T;
};

__global__ __launch_bounds__(kBlock) void k_up1(UpArgs g) {
  __shared__ float s_p[kRPG * 4];
  if (blockIdx.x == 0) zero_tickets(g.ctr, g.T);
  int n = *g.count;
  n = n < 0 ? 0 : (n > g.F ? g.F : n);
  if ((int)blockIdx.x * kRPG >= n) return;  // (uniform)
  const UpSlices o = up_slices(g.d);
  uint4 xv[kUQ], w[kRPG][kUQ];
  x_slices(g.x, g.d, o, xv);
  for (int k0 = blockIdx.x * kRPG; k0 < n; k0 += gridDim.x * kRPG) {
    int ids[kRPG];
#pragma unroll
    for (int r = 0; r < kRPG; ++r) {
      const int v = k0 + r < n ? __builtin_amdgcn_readfirstlane(g.idx[k0 + r]) : -1;
      ids[r] = (unsigned)v < (unsigned)g.F ? v : -1;
    }
    up_rows_load(g.w_up, g.d, ids, o, w);
    up_rows_finish(w, xv, ids, g.b_up, g.a, s_p);
  }
}

// =========================================================================================
// The down projection of one (column tile t, split s): a_i W_dT[i][t*kTile, (t+1)*kTile) summed over
// the split's neurons.  The split's id sequence is built in segments of kBlock * kSeg candidates
// (list entries, or the mask words' bit s) by a block prefix sum; its k-th id goes to wave k mod 4,
// which accumulates its ids in sequence order (8 columns per lane, kDnRB rows in flight).  The four
// wave sums are added in wave order into the split's partial part[s][cols]; then the tile's
// completion ticket, and the last workgroup of the tile adds the S partials in split order (after
// b_down, or onto y) and re-arms the ticket.
//   LIST:  ids from a list (entries with i mod S == s, in list order): FFN call
//   !LIST: ids from the mask words, ascending: layer call

struct DnArgs {
  const uint32_t* masks;  // !LIST: kept bits (bit b of word q: neuron 32 q + b)
  int nq;
  const int32_t* idx;     // LIST
  const int32_t* count;
  const float* a;
  const void* w_dT;       // fp16 rows of d, or 4-bit rows of d/2 bytes
  const uint16_t* s_dT;   // 4-bit: fp16 scales [F][d/128]
  const float* b_down;
  float* part;            // [S][d]
  uint32_t* ctr;          // [T] tickets, kTicketStride apart
  float* y;
  int d, F, T, accumulate;
};

template <bool LIST, bool I4>
__device__ __forceinline__ void dn_split(const DnArgs& g, int t, int s) {
  constexpr int CPL = I4 ? kCPL4 : 8;    // output columns per lane
  constexpr int TILE = kWave * CPL;      // kTile (fp16) or kTile4 (4-bit)
  constexpr int NPT = TILE / kBlock;     // columns per thread in the partial and the final sum
  constexpr int RB = I4 ? kDn4RB : kDnRB;
  static_assert(TILE == (I4 ? kTile4 : kTile) && NPT % 2 == 0, "tile shape");
  static_assert(kBlock * kSeg <= (kBlock / kWave) * TILE, "the id list and the wave sums share one buffer");
  __shared__ float s_buf[(kBlock / kWave) * TILE];  // the segment's ids, then (after the rows) the four wave sums
  __shared__ int s_red[kBlock / kWave];
  __shared__ int s_last;
  int* s_i = reinterpret_cast<int*>(s_buf);
  float (*s_acc)[TILE] = reinterpret_cast<float (*)[TILE]>(s_buf);
  constexpr int S = kMaxSplits;
  const int lane = wave_lane(), wv = wave_id();
  const int col = t * TILE + lane * CPL;
  const bool colok = col < g.d;
  // fp16: the lane's 16-byte slice of a row; 4-bit: its 8 bytes and the scale of its 128-column group
  const char* wd = static_cast<const char*>(g.w_dT) + (size_t)col * 2;
  const size_t rb = (size_t)g.d * 2;
  const uint32_t rowb4 = (uint32_t)g.d / 2, scb4 = (uint32_t)(g.d / 128) * 2;
  const uint32_t woff4 = colok ? (uint32_t)col / 2 : kOob, soff4 = colok ? (uint32_t)(col / 128) * 2 : kOob;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  // candidates: list positions, or the words q = s / 32 + kSW k (bit s % 32)
  int ncand;
  if constexpr (LIST) {
    const int n = *g.count;
    ncand = n < 0 ? 0 : (n > g.F ? g.F : n);
  } else {
    const int q0 = s >> 5;
    ncand = q0 < g.nq ? (g.nq - q0 + kSW - 1) / kSW : 0;
  }
  int base = 0;  // ids of the split's sequence before this segment
  for (int seg = 0; seg < ncand; seg += kBlock * kSeg) {
    const int k0 = seg + threadIdx.x * kSeg;
    int ids[kSeg];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kSeg; ++u) {
      const int k = k0 + u;
      int id = -1;
      if constexpr (LIST) {
        const int v = g.idx[k < ncand ? k : 0];  // (unconditional load; idx holds >= 1 entry)
        id = (k < ncand && (unsigned)v < (unsigned)g.F && (v % S) == s) ? v : -1;
      } else {
        const int q = (s >> 5) + kSW * k;
        const uint32_t wbits = g.masks[k < ncand ? q : 0];  // (unconditional load)
        id = (k < ncand && ((wbits >> (s & 31)) & 1u)) ? q * 32 + (s & 31) : -1;
      }
      ids[u] = id;
      c += id >= 0;
    }
    int ns;
    int at = block_excl(c, s_red, ns);
#pragma unroll
    for (int u = 0; u < kSeg; ++u)
      if (ids[u] >= 0) s_i[at++] = ids[u];
    __syncthreads();
    // this wave's ids of the segment: sequence positions base + jj with (base + jj) % 4 == wv
    const int j0 = (wv - (base & 3) + 4) & 3;
    for (int j = j0; j < ns; j += 4 * RB) {
      if constexpr (I4) {
        constexpr int NW = CPL / 8;  // 32-bit words of nibbles per lane and row
        uint32_t wr[RB][NW];
        uint32_t sc[RB];
        float av[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int jj = j + 4 * r;
          const int i = jj < ns ? s_i[jj] : -1;
          const __amdgpu_buffer_rsrc_t rr = row_rsrc(g.w_dT, i, rowb4);
          if constexpr (NW == 2) {
            const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rr, woff4, 0, kNT));
            wr[r][0] = v.x;
            wr[r][NW - 1] = v.y;
          } else {
            wr[r][0] = __builtin_amdgcn_raw_buffer_load_b32(rr, woff4, 0, kNT);
          }
          sc[r] = __builtin_amdgcn_raw_buffer_load_b16(row_rsrc(g.s_dT, i, scb4), soff4, 0, 0);
          av[r] = *(i >= 0 ? g.a + i : s_zero_f);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float f = av[r] * h2f(sc[r]);
#pragma unroll
          for (int q = 0; q < NW; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[8 * q + e] = fmaf(f, i4_elem(wr[r][q], e), acc[8 * q + e]);
        }
      } else {
        uint4 wr[RB];
        float av[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int jj = j + 4 * r;
          const bool ok = jj < ns;
          const int i = ok ? s_i[jj] : 0;
          wr[r] = ldz16_nt(wd + (size_t)i * rb, ok && colok);
          av[r] = *(ok ? g.a + i : s_zero_f);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const uint32_t ww[4] = {wr[r].x, wr[r].y, wr[r].z, wr[r].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            acc[2 * h] = fmaf(av[r], h2f(ww[h] & 0xffffu), acc[2 * h]);
            acc[2 * h + 1] = fmaf(av[r], h2f(ww[h] >> 16), acc[2 * h + 1]);
          }
        }
      }
    }
    base += ns;
    __syncthreads();  // s_i and s_red are rewritten by the next segment
  }
  // the split's partial: the four wave sums in wave order
#pragma unroll
  for (int c = 0; c < CPL; ++c) s_acc[wv][lane * CPL + c] = acc[c];
  __syncthreads();
  const int c0 = NPT * threadIdx.x;
  const int gc = t * TILE + c0;  // d % 8 == 0 (fp16), d % 128 == 0 (4-bit): gc < d implies gc + NPT <= d
  if (gc < g.d) {
    float v[NPT];
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      v[e] = s_acc[0][c0 + e];
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) v[e] += s_acc[w][c0 + e];
    }
#pragma unroll
    for (int e = 0; e < NPT; e += 2) st_dev64(g.part + (size_t)s * g.d + gc + e, v[e], v[e + 1]);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* tk = g.ctr + t * kTicketStride;
    const bool last = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1);
    if (last) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // every split has arrived
    s_last = last;
  }
  __syncthreads();
  if (!s_last || gc >= g.d) return;
  // the tile's last workgroup: y = (y +) (b_down + sum of the S partials in split order)
  float tv[NPT];
#pragma unroll
  for (int e = 0; e < NPT; ++e) tv[e] = g.b_down ? g.b_down[gc + e] : 0.f;
  constexpr int kFin = 16;  // splits per round: 16 NPT / 2 partial pairs in flight
#pragma unroll
  for (int s0 = 0; s0 < S; s0 += kFin) {
    uint64_t v[kFin][NPT / 2];
#pragma unroll
    for (int u = 0; u < kFin; ++u)
#pragma unroll
      for (int e = 0; e < NPT / 2; ++e) v[u][e] = ld_dev64(g.part + (size_t)(s0 + u) * g.d + gc + 2 * e);
#pragma unroll
    for (int u = 0; u < kFin; ++u)
#pragma unroll
      for (int e = 0; e < NPT / 2; ++e) {
        tv[2 * e] += __uint_as_float((uint32_t)v[u][e]);
        tv[2 * e + 1] += __uint_as_float((uint32_t)(v[u][e] >> 32));
      }
  }
  float* yp = g.y + gc;
#pragma unroll
  for (int e = 0; e < NPT; ++e) yp[e] = g.accumulate ? yp[e] + tv[e] : tv[e];
}

// k_dn: the down projection, workgroup (t, s) = blockIdx % T, blockIdx / T; in mask mode one more
// workgroup (the last) writes the ascending list of kept neurons and its length
__device__ __forceinline__ void write_list(const uint32_t* masks, int nq, int32_t* idx, int32_t* count);

struct DnList {
  int32_t* idx;
  int32_t* count;
};

template <bool LIST, bool I4>
__global__ __launch_bounds__(kBlock) void k_dn(DnArgs g, DnList out) {
  const int b = blockIdx.x;
  if (!LIST && b == g.T * kMaxSplits) {
    write_list(g.masks, g.nq, out.idx, out.count);
    return;
  }
  dn_split<LIST, I4>(g, b % g.T, b / g.T);
}

// the ascending list of kept neurons and its length from the mask words, in rounds of kBlock * kLW
// words: thread t takes the round's words [kLW t, kLW t + kLW)
__device__ __forceinline__ void write_list(const uint32_t* masks, int nq, int32_t* idx, int32_t* count) {
  __shared__ int s_red[kBlock / kWave];
  constexpr int kLW = 4;
  int base = 0;
  for (int r0 = 0; r0 < nq; r0 += kBlock * kLW) {
    const int q0 = r0 + threadIdx.x * kLW;
    uint32_t wv[kLW];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kLW; ++u) {
      wv[u] = masks[q0 + u < nq ? q0 + u : 0];
      if (q0 + u >= nq) wv[u] = 0u;
      c += __popc(wv[u]);
    }
    int total;
    int at = base + block_excl(c, s_red, total);
#pragma unroll
    for (int u = 0; u < kLW; ++u) {
      uint32_t m = wv[u];
      while (m != 0u) {
        idx[at++] = (q0 + u) * 32 + (int)__builtin_ctz(m);
        m &= m - 1u;
      }
    }
    base += total;
    __syncthreads();  // s_red is rewritten by the next round
  }
  if (threadIdx.x == 0) *count = base;
}

// =========================================================================================
// 4-bit weights at one token (ReLU): the same pipeline as fp16 (k_qu's up rows and k_up1_i4 share
// the 4-bit up-row code; k_dn<., true> takes 16 columns, 8 bytes, of each row per lane).  Row i of
// W_up and of W_dT holds d/2 bytes (element 2j in the low nibble of byte j, two's complement) and
// d/128 fp16 scales, one per 128 consecutive elements.


struct Up4Args {
  const int32_t* idx;
  const int32_t* count;
  const uint8_t* w_up;
  const uint16_t* s_up;
  const float* b_up;
  const _Float16* x;
  float* a;
  uint32_t* ctr;
  int F, d, T;
};

// The 4-bit up rows in k_up1's scheme with 32-element slices: wave w covers the quarter
// [w S4, w S4 + S4) of a row's slices and lane L its slices w S4 + L + 64 u (u < kUQ4).  A slice
// lies in one scale group, so its dot product (exact fp16 products, fp32 sums) takes one scale;
// the row's value is then committed as in up_rows_finish.  The lane's x slices are loaded and
// paired (pair_x8) once per workgroup.
struct Up4Slices {
  uint32_t woff[kUQ4], xoff[kUQ4], soff[kUQ4];  // byte offsets in a weight row, x, a scale row (kOob: none)
};

__device__ __forceinline__ Up4Slices up4_slices(int d) {
  const int nsl = d / 32, S4 = (nsl + 3) / 4;
  const int w = wave_id(), L = wave_lane();
  Up4Slices o;
#pragma unroll
  for (int u = 0; u < kUQ4; ++u) {
    const int k = L + kWave * u, sl = w * S4 + k;
    const bool ok = k < S4 && sl < nsl;
    o.woff[u] = ok ? (uint32_t)sl * 16 : kOob;
    o.xoff[u] = ok ? (uint32_t)sl * 64 : kOob;
    o.soff[u] = ok ? (uint32_t)(sl / 4) * 2 : kOob;
  }
  return o;
}

__device__ __forceinline__ void x4_slices(const _Float16* __restrict__ x, int d, const Up4Slices& o,
                                          uint4 (&px)[kUQ4][4]) {
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(x), 0, d * 2, kRsrcWord3);
#pragma unroll
  for (int u = 0; u < kUQ4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) px[u][v] = bload16(xr, o.xoff[u] == kOob ? kOob : o.xoff[u] + 16 * v);
#pragma unroll
  for (int u = 0; u < kUQ4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) px[u][v] = pair_x8(px[u][v]);
}

__device__ __forceinline__ void up4_rows_load(const uint8_t* __restrict__ w_up, const uint16_t* __restrict__ s_up,
                                              int d, const int (&ids)[kRPG], const Up4Slices& o,
                                              uint4 (&wq)[kRPG][kUQ4], uint32_t (&sc)[kRPG][kUQ4]) {
  const uint32_t rowb = (uint32_t)d / 2, scb = (uint32_t)(d / 128) * 2;
#pragma unroll
  for (int r = 0; r < kRPG; ++r) {
    const __amdgpu_buffer_rsrc_t wr = row_rsrc(w_up, ids[r], rowb);
    const __amdgpu_buffer_rsrc_t sr = row_rsrc(s_up, ids[r], scb);
#pragma unroll
    for (int u = 0; u < kUQ4; ++u) {
      wq[r][u] = bload16_nt(wr, o.woff[u]);
      sc[r][u] = __builtin_amdgcn_raw_buffer_load_b16(sr, o.soff[u], 0, 0);
    }
  }
}

__device__ __forceinline__ void up4_rows_finish(const uint4 (&wq)[kRPG][kUQ4], const uint32_t (&sc)[kRPG][kUQ4],
                                                const uint4 (&px)[kUQ4][4], const int (&ids)[kRPG],
                                                const float* __restrict__ b_up, float* __restrict__ a, float* s_p) {
  const int lane = wave_lane(), wv = wave_id();
#pragma unroll
  for (int r = 0; r < kRPG; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kUQ4; ++u) {
      float t = 0.f;
      t = dot8_i4(wq[r][u].x, px[u][0], t);
      t = dot8_i4(wq[r][u].y, px[u][1], t);
      t = dot8_i4(wq[r][u].z, px[u][2], t);
      t = dot8_i4(wq[r][u].w, px[u][3], t);
      acc = fmaf(t, h2f(sc[r][u]), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) s_p[r * 4 + wv] = acc;
  }
  __syncthreads();
  if (threadIdx.x < kRPG) {
    const int r = threadIdx.x;
    int i = -1;
#pragma unroll
    for (int k = 0; k < kRPG; ++k)
      if (k == r) i = ids[k];
    if (i >= 0) {
      const float z = ((s_p[r * 4] + s_p[r * 4 + 1]) + s_p[r * 4 + 2]) + s_p[r * 4 + 3];
      const float v = z + (b_up ? b_up[i] : 0.f);
      a[i] = v > 0.f ? v : 0.f;
    }
  }
  __syncthreads();
}

// k_up1_i4: a_i for the neurons of a given list with 4-bit rows (FFN call), kRPG list entries per
// workgroup at a time; entries outside [0, F) are skipped.  Workgroup 0 zeroes k_dn's tickets.
__global__ __launch_bounds__(kBlock) void k_up1_i4(Up4Args g) {
  __shared__ float s_p[kRPG * 4];
  if (blockIdx.x == 0) zero_tickets(g.ctr, g.T);
  int n = *g.count;
  n = n < 0 ? 0 : (n > g.F ? g.F : n);
  if ((int)blockIdx.x * kRPG >= n) return;  // (uniform)
  const Up4Slices o = up4_slices(g.d);
  uint4 px[kUQ4][4];
  x4_slices(g.x, g.d, o, px);
  for (int k0 = blockIdx.x * kRPG; k0 < n; k0 += gridDim.x * kRPG) {
    int ids[kRPG];
#pragma unroll
    for (int r = 0; r < kRPG; ++r) {
      const int v = k0 + r < n ? __builtin_amdgcn_readfirstlane(g.idx[k0 + r]) : -1;
      ids[r] = (unsigned)v < (unsigned)g.F ? v : -1;
    }
    uint4 wq[kRPG][kUQ4];
    uint32_t sc[kRPG][kUQ4];
    up4_rows_load(g.w_up, g.s_up, g.d, ids, o, wq, sc);
    up4_rows_finish(wq, sc, px, ids, g.b_up, g.a, s_p);
  }
}

// =========================================================================================
// k_h1: h = A x at one token without the LayerNorm, one single-wave workgroup per row of A: the
// lane's 16-byte slices of the row and of x (u < UN, rows of up to UN * 512 fp16) are all requested
// at once and x is read straight from L2 (no LDS copy, no barrier), so r small workgroups keep the
// whole of A in flight.  The same per-lane order and wave sum as the small-batch k_h: the same h.
// It also zeroes the nzero words at zero (the mask words k_qu ORs its bits into).
template <int UN>
__global__ __launch_bounds__(kWave) void k_h1(const _Float16* __restrict__ A, const _Float16* __restrict__ x, int d,
                                              float* __restrict__ h, uint32_t* __restrict__ zero, int nzero) {
  for (int k = blockIdx.x * kWave + threadIdx.x; k < nzero; k += gridDim.x * kWave) zero[k] = 0u;
  const int j = blockIdx.x, lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t ra = row_rsrc(A, j, (uint32_t)d * 2);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(x), 0, d * 2, kRsrcWord3);
  uint4 w[UN], xv[UN];
  // slice u of the row and of x requested together: loads return in issue order, so the dot products
  // follow the data in (OPT-175B-shaped 4-bit layer, 24 slices: 52.9 -> 52.5 us per layer)
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    w[u] = bload16_nt(ra, (uint32_t)(u * kWave + lane) * 16);
    xv[u] = bload16(rx, (uint32_t)(u * kWave + lane) * 16);
  }
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < UN; ++u)
    if ((u * kWave + lane) * 8 < d) acc = dot8_f16(w[u], xv[u], acc);
  acc = wave_sum(acc);
  if (lane == 0) h[j] = acc;
}

// =========================================================================================
// k_qu: the logits of chunk q (16 neurons interleaved within a block of kIlv chunks: the logits
// kernel's arithmetic, the same bits as psffn_predict), their bits ORed into the mask words (zeroed by
// the kernel before), then the up rows of the kept ones, kRPG at a time by the whole workgroup.  The
// interleave spreads the hot neurons of a hot-first layer (low indices) over the first block's
// chunks, so no workgroup is left with a chunk of 16 hot rows.

struct QuArgs {
  const void* Q;
  const float* c;
  const float* h;
  float* logits;
  uint32_t* masks;
  const void* w_up;      // fp16 rows of d, or 4-bit rows of d/2 bytes
  const uint16_t* s_up;  // 4-bit: fp16 scales [F][d/128]
  const float* b_up;  // or null
  const _Float16* x;
  float* a;           // [F] activations by neuron
  uint32_t* ctr;      // k_dn's tickets (zeroed here)
  int r, F, d, NC, n_hot, T;
  float thr;
};

template <int RV, bool I4>
__global__ __launch_bounds__(kBlock) void k_qu(QuArgs g) {
  const int q = blockIdx.x;
  if (q == 0) zero_tickets(g.ctr, g.T);
  const uint32_t m = q_chunk<St::F16, 1, RV, 4, kIlv>(g.Q, g.c, g.h, g.r, g.F, g.thr, 1, g.logits, g.n_hot, q,
                                                       g.NC);
  if (threadIdx.x < 16 && ((m >> threadIdx.x) & 1u)) {
    const int i = chunk_neuron<kIlv, 4>(q, g.NC, (int)threadIdx.x);
    __hip_atomic_fetch_or(g.masks + (i >> 5), 1u << (i & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (m == 0u) return;  // (uniform: every thread holds the same bits)
  __shared__ float s_p[kRPG * 4];
  const uint32_t mu = __builtin_amdgcn_readfirstlane(m);
  const int nset = __popc(mu);
  if constexpr (I4) {
    const Up4Slices o = up4_slices(g.d);
    uint4 px[kUQ4][4], wq[kRPG][kUQ4];
    uint32_t sc[kRPG][kUQ4];
    x4_slices(g.x, g.d, o, px);
    for (int j0 = 0; j0 < nset; j0 += kRPG) {
      int ids[kRPG];
#pragma unroll
      for (int r = 0; r < kRPG; ++r)
        ids[r] = j0 + r < nset ? chunk_neuron<kIlv, 4>(q, g.NC, nth_bit(mu, j0 + r)) : -1;
      up4_rows_load(static_cast<const uint8_t*>(g.w_up), g.s_up, g.d, ids, o, wq, sc);
      up4_rows_finish(wq, sc, px, ids, g.b_up, g.a, s_p);
    }
  } else {
    const UpSlices o = up_slices(g.d);
    uint4 xv[kUQ], w[kRPG][kUQ];
    x_slices(g.x, g.d, o, xv);
    for (int j0 = 0; j0 < nset; j0 += kRPG) {
      int ids[kRPG];
#pragma unroll
      for (int r = 0; r < kRPG; ++r)
        ids[r] = j0 + r < nset ? chunk_neuron<kIlv, 4>(q, g.NC, nth_bit(mu, j0 + r)) : -1;
      up_rows_load(static_cast<const _Float16*>(g.w_up), g.d, ids, o, w);
      up_rows_finish(w, xv, ids, g.b_up, g.a, s_p);
    }
  }
}

int tiles_of(int d) { return (d + kTile - 1) / kTile; }

// scratch after the mask words: activations [F], partials [S][d], tickets (T lines), h [r]
struct StreamBufs {
  float* a;
  float* part;
  uint32_t* ctr;   // T tickets, kTicketStride words apart
  float* h;
};

size_t ctr_words(int d) { return (size_t)tiles_of(d) * kTicketStride; }

StreamBufs stream_bufs(void* ws, int F, int d) {
  char* base = static_cast<char*>(ws) + state_layout(F).scratch;
  StreamBufs b;
  b.a = reinterpret_cast<float*>(base);
  base += round256((size_t)F * 4);
  b.part = reinterpret_cast<float*>(base);
  base += round256((size_t)kMaxSplits * d * 4);
  b.ctr = reinterpret_cast<uint32_t*>(base);
  base += round256(ctr_words(d) * 4);
  b.h = reinterpret_cast<float*>(base);
  return b;
}

template <int RV>
void qu_launch(const QuArgs& g, bool i4, hipStream_t s) {
  if (i4) k_qu<RV, true><<<g.NC, kBlock, 0, s>>>(g);
  else k_qu<RV, false><<<g.NC, kBlock, 0, s>>>(g);
}

// the down projection's column tiles (and ticket lines): kTile columns for fp16 rows, kTile4 for 4-bit
int dn_tiles(const psffn_ffn& W) { return W.dt == PSFFN_I4G128 ? (W.d + kTile4 - 1) / kTile4 : tiles_of(W.d); }

}  // namespace

size_t stream_scratch(int r, int F, int d) {
  return round256((size_t)F * 4) + round256((size_t)kMaxSplits * d * 4) + round256(ctr_words(d) * 4) +
         round256((size_t)r * 4);
}

hipError_t launch_h1(const psffn_predictor& P, const void* x, float* h, hipStream_t s) {
  if (P.dt != PSFFN_F16 || P.d > 24 * kWave * 8) return hipErrorNotSupported;
  const _Float16* A = static_cast<const _Float16*>(P.A);
  const _Float16* xv = static_cast<const _Float16*>(x);
  if (P.d <= kUQ * 4 * kWave * 8) k_h1<kUQ * 4><<<P.r, kWave, 0, s>>>(A, xv, P.d, h, nullptr, 0);
  else k_h1<24><<<P.r, kWave, 0, s>>>(A, xv, P.d, h, nullptr, 0);
  return hipGetLastError();
}

bool stream_ffn_fits(const psffn_ffn& W, int B) {
  return B == 1 && W.dt == PSFFN_F16 && W.act == PSFFN_RELU && W.d % 8 == 0 && W.d <= kUQ * 4 * kWave * 8;
}

bool stream_ffn_i4_fits(const psffn_ffn& W, int B) {
  return B == 1 && W.dt == PSFFN_I4G128 && W.act == PSFFN_RELU && W.d % 128 == 0 && W.d <= kUQ4 * 4 * kWave * 32;
}

bool stream_layer_fits(const psffn_predictor& P, const psffn_ffn& W, int B, bool ln) {
  if (!(stream_ffn_fits(W, B) || stream_ffn_i4_fits(W, B)) || P.dt != PSFFN_F16 || P.F != W.F || P.d != W.d)
    return false;
  const int rv = (P.r + kWave * 8 - 1) / (kWave * 8);
  if (rv < 1 || rv > 4 || (W.F + 31) / 32 > kMaxWords) return false;
  if (ln && ln_k(P.d) == 0) return false;
  return true;
}

hipError_t launch_ffn_stream(const psffn_ffn& W, const void* x, const int32_t* idx, const int32_t* count, float* y,
                             int accumulate, void* ws, hipStream_t s) {
  if (stream_ffn_i4_fits(W, 1)) {
    const StreamBufs bf = stream_bufs(ws, W.F, W.d);
    Up4Args u{};
    u.idx = idx;
    u.count = count;
    u.w_up = static_cast<const uint8_t*>(W.w_up);
    u.s_up = static_cast<const uint16_t*>(W.s_up);
    u.b_up = W.b_up;
    u.x = static_cast<const _Float16*>(x);
    u.a = bf.a;
    u.ctr = bf.ctr;
    u.F = W.F;
    u.d = W.d;
    u.T = dn_tiles(W);
    const int grid = W.F < kRPG * 1024 ? (W.F + kRPG - 1) / kRPG : 1024;
    k_up1_i4<<<grid, kBlock, 0, s>>>(u);
    DnArgs g{};
    g.idx = idx;
    g.count = count;
    g.a = bf.a;
    g.w_dT = W.w_dT;
    g.s_dT = static_cast<const uint16_t*>(W.s_dT);
    g.b_down = W.b_down;
    g.part = bf.part;
    g.ctr = bf.ctr;
    g.y = y;
    g.d = W.d;
    g.F = W.F;
    g.T = dn_tiles(W);
    g.accumulate = accumulate;
    k_dn<true, true><<<(unsigned)(g.T * kMaxSplits), kBlock, 0, s>>>(g, DnList{});
    return hipGetLastError();
  }
  if (!stream_ffn_fits(W, 1)) return hipErrorNotSupported;
  const StreamBufs bf = stream_bufs(ws, W.F, W.d);
  UpArgs u{};
  u.idx = idx;
  u.count = count;
  u.w_up = static_cast<const _Float16*>(W.w_up);
  u.b_up = W.b_up;
  u.x = static_cast<const _Float16*>(x);
  u.a = bf.a;
  u.ctr = bf.ctr;
  u.F = W.F;
  u.d = W.d;
  u.T = tiles_of(W.d);
  const int grid = W.F < kRPG * 1024 ? (W.F + kRPG - 1) / kRPG : 1024;
  k_up1<<<grid, kBlock, 0, s>>>(u);
  DnArgs g{};
  g.idx = idx;
  g.count = count;
  g.a = bf.a;
  g.w_dT = W.w_dT;
  g.b_down = W.b_down;
  g.part = bf.part;
  g.ctr = bf.ctr;
  g.y = y;
  g.d = W.d;
  g.F = W.F;
  g.T = tiles_of(W.d);
  g.accumulate = accumulate;
  k_dn<true, false><<<(unsigned)(g.T * kMaxSplits), kBlock, 0, s>>>(g, DnList{});
  return hipGetLastError();
}

hipError_t launch_layer_stream(const psffn_predictor& P, const psffn_ffn& W, const void* x, float thr, int32_t* idx,
                               int32_t* count, float* logits, float* y, int accumulate, void* ws, hipStream_t s,
                               int n_hot, const LnArgs& ln) {
  if (!stream_layer_fits(P, W, 1, ln.xres != nullptr)) return hipErrorNotSupported;
  const StreamBufs bf = stream_bufs(ws, W.F, W.d);
  uint32_t* masks = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + state_layout(P.F).masks);
  const int nq = (P.F + 31) / 32;
  const bool i4 = W.dt == PSFFN_I4G128;
  // the first kernel zeroes the mask words (k_qu ORs its bits into them); k_h1 holds rows of up to
  // 24 * 512 elements, longer rows (4-bit layers, d <= 16384) and the LayerNorm take k_h
  if (ln.xres == nullptr && P.d <= kUQ * 4 * kWave * 8) {
    k_h1<kUQ * 4><<<P.r, kWave, 0, s>>>(static_cast<const _Float16*>(P.A), static_cast<const _Float16*>(x), P.d, bf.h,
                                         masks, nq);
  } else if (ln.xres == nullptr && P.d <= 24 * kWave * 8) {
    k_h1<24><<<P.r, kWave, 0, s>>>(static_cast<const _Float16*>(P.A), static_cast<const _Float16*>(x), P.d, bf.h,
                                   masks, nq);
  } else {
    const hipError_t e = launch_h_f16_b1(P, x, bf.h, ln, s, masks, nq, nullptr, 0);
    if (e != hipSuccess) return e;
  }
  QuArgs q{};
  q.Q = P.Q;
  q.c = P.c;
  q.h = bf.h;
  q.logits = logits;
  q.masks = masks;
  q.w_up = W.w_up;
  q.s_up = static_cast<const uint16_t*>(W.s_up);
  q.b_up = W.b_up;
  q.x = static_cast<const _Float16*>(ln.xres ? static_cast<const void*>(ln.hout) : x);
  q.a = bf.a;
  q.ctr = bf.ctr;
  q.T = dn_tiles(W);
  q.r = P.r;
  q.F = P.F;
  q.d = P.d;
  q.NC = (P.F + 15) / 16;
  q.n_hot = n_hot;
  q.thr = thr;
  const int rv = (P.r + kWave * 8 - 1) / (kWave * 8);
  if (rv == 1) qu_launch<1>(q, i4, s);
  else if (rv == 2) qu_launch<2>(q, i4, s);
  else if (rv == 3) qu_launch<3>(q, i4, s);
  else qu_launch<4>(q, i4, s);
  DnArgs g{};
  g.masks = masks;
  g.nq = nq;
  g.a = bf.a;
  g.w_dT = W.w_dT;
  g.s_dT = static_cast<const uint16_t*>(W.s_dT);
  g.b_down = W.b_down;
  g.part = bf.part;
  g.ctr = bf.ctr;
  g.y = ln.xres ? const_cast<float*>(ln.xres) : y;
  g.d = W.d;
  g.F = W.F;
  g.T = dn_tiles(W);
  g.accumulate = ln.xres ? 1 : accumulate;
  if (i4) k_dn<false, true><<<(unsigned)(g.T * kMaxSplits + 1), kBlock, 0, s>>>(g, DnList{idx, count});
  else k_dn<false, false><<<(unsigned)(g.T * kMaxSplits + 1), kBlock, 0, s>>>(g, DnList{idx, count});
  return hipGetLastError();
}

}  // namespace psffn

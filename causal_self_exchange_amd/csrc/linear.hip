// Linear Relation forward ("Ask Self, Ask Others: Relation Is All You Need",
// Sec. 5.2 Eq. (15)-(17), App. A.4) in chunk-parallel form.
//
// Per head: S_t = sigmoid(p1_t . p2_t / (tau sqrt(d_h))), q_t = p1_t / |p1_t|,
// k_t = p2_t / |p2_t|, and the recurrent state C (d_h x d_h, rows along the
// relation coordinate, columns along the information channel):
//   C-_t = Diag(alpha_t) C_{t-1};  Y_t = I_t + S_t (C-_t)^T q_t;  C_t = C-_t + S_t k_t I_t^T.
// With 64-token chunks and b_t = sum of log alpha_u over the chunk up to t
// (per channel), the state entering chunk c is Cin_c and
//   Y_t = I_t + S_t Cin_c^T (q_t o e^{b_t})
//             + S_t sum_{j<t in chunk} S_j (sum_r q_{t,r} k_{j,r} e^{b_{t,r} - b_{j,r}}) I_j
//   Cin_{c+1} = Diag(e^{b_last}) Cin_c + sum_j S_j (k_j o e^{b_last - b_j}) I_j^T.
// Every exponent above is <= 0, so any retention in (0, 1] is safe.
// Chunks are taken in groups of consecutive chunks of one head, and only one
// state per group passes through memory. Three kernels: chunk (per group, its
// chunks in order with the state accumulators in registers: the group's
// contribution and decay), scan (the elementwise recurrence over groups, one
// thread per state element), output (per group, its chunks in order: Y, with
// the entering state stepped from chunk to chunk on chip). Arithmetic is fp32
// throughout; with bf16 inputs the large products (the contributions K^T I,
// the output's at I, Qt Cin and state update, and its intra-chunk sub-blocks)
// run on bf16 MFMA with every fp32 operand split into a bf16 pair (I itself
// is exact in bf16), which carries it to about 2^-17 relative.
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

constexpr int kL = kLinChunk;          // tokens per chunk
constexpr int kChunkThreads = 512;     // chunk kernel: 8 waves, 66 KB of LDS
constexpr int kOutThreads = 512;       // output kernel: 8 waves, 152 KB of LDS
constexpr int kScanThreads = 256;
static_assert(kL == 64, "the output kernel's sub-block pairs assume 4 blocks of 16 rows");
// Decay prefixes are kept in base 2 (b2 = log2 of the retention product), so
// every decay factor is one hardware 2^x. A diagonal 16-row block of the
// intra-chunk weights factors through its middle row when every exponent of
// the two factors lies in [-57, 57] (about e^+-40): the factors and their
// products then stay normal fp32 numbers.
constexpr float kFactorBound = 57.0f;
__device__ __forceinline__ float pow2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// x = hi + lo + O(2^-17 |x|): hi is x rounded to bf16 (nearest even), lo the
// exact fp32 remainder x - hi rounded to bf16. A product of two split operands
// is taken as hi hi + hi lo + lo hi (the dropped lo lo is below 2^-16 of it),
// on bf16 MFMA with fp32 accumulation.
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8v& hi, bf16x8v& lo) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    hi[u] = (__bf16)x[u];
    lo[u] = (__bf16)(x[u] - (float)hi[u]);
  }
}

// bf16 operand tiles in LDS: row `row` of 8-element (16-byte) chunks, the
// chunk index XOR-swizzled with a function of the row so that the MFMA
// operand reads (32 rows, one chunk each) spread over the banks. Rows of 8
// chunks (64 elements) and of 16 chunks (128 elements).
__device__ __forceinline__ int sw8(int row, int c) { return row * 128 + 16 * (c ^ ((row >> 1) & 7)); }
__device__ __forceinline__ int sw16(int row, int c) { return row * 256 + 16 * (c ^ (row & 15)); }
// Rows of D elements (D / 8 chunks).
template <int D>
__device__ __forceinline__ int swd(int row, int c) {
  if constexpr (D == 128) return sw16(row, c);
  else if constexpr (D == 64) return sw8(row, c);
  else return row * 64 + 16 * (c ^ ((row >> 2) & 3));
}
__device__ __forceinline__ bf16x8v lds_bf16x8(const char* base, int off) {
  return *reinterpret_cast<const bf16x8v*>(base + off);
}

template <typename Tin>
__device__ __forceinline__ float ld_val(const Tin* p, size_t i) { return to_f32(p[i]); }

// A chunk's rows (rows >= `rows` give 0) in registers: NT threads (tid = the
// thread's index) issue every 16-byte load before any is used, so one memory
// latency covers the chunk.
template <int NT, typename Tin, int D>
struct Staged {
  static constexpr int kVec = 16 / (int)sizeof(Tin);   // elements per 16-byte load
  static constexpr int kTot = kL * D / kVec;            // loads per chunk
  static constexpr int kN = (kTot + NT - 1) / NT;       // loads per thread
  static_assert(kL * D % kVec == 0, "whole loads per row");
  u32x4v v[kN];

  __device__ __forceinline__ void load(const Tin* src, int rows, int tid) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = tid + i * NT, e = idx * kVec;
      v[i] = (idx < kTot && e / D < rows) ? *reinterpret_cast<const u32x4v*>(src + e) : u32x4v{0u, 0u, 0u, 0u};
    }
  }
  // Load i as fp32: row (tid + i NT) / (D / kVec), kVec consecutive channels.
  __device__ __forceinline__ void unpack(int i, float (&x)[kVec]) const {
    if constexpr (sizeof(Tin) == 2) {
      typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
      const bf16x8v b = __builtin_bit_cast(bf16x8v, v[i]);
#pragma unroll
      for (int u = 0; u < kVec; ++u) x[u] = (float)b[u];
    } else {
#pragma unroll
      for (int u = 0; u < kVec; ++u) x[u] = __uint_as_float(v[i][u]);
    }
  }
  // Into an fp32 LDS array, row-major [t][r] (ld = row stride) or
  // channel-major [r][t].
  template <bool kChannelMajor>
  __device__ __forceinline__ void store(float* dst, int ld, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = tid + i * NT, e = idx * kVec;
      if (idx >= kTot) break;
      const int t = e / D, r0 = e % D;
      float x[kVec];
      unpack(i, x);
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
        if (kChannelMajor) dst[(r0 + u) * ld + t] = x[u];
        else dst[t * ld + r0 + u] = x[u];
      }
    }
  }
  // As store, each load's elements multiplied by sc[i] first.
  template <bool kChannelMajor>
  __device__ __forceinline__ void store_scaled(float* dst, int ld, int tid, const float (&sc)[kN]) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = tid + i * NT, e = idx * kVec;
      if (idx >= kTot) break;
      const int t = e / D, r0 = e % D;
      float x[kVec];
      unpack(i, x);
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
        if (kChannelMajor) dst[(r0 + u) * ld + t] = x[u] * sc[i];
        else dst[t * ld + r0 + u] = x[u] * sc[i];
      }
    }
  }
  // bf16 rows (exact) into a channel-major bf16 tile: element (t, r) at
  // sw8(r, t / 8) + 2 (t % 8), i.e. the tokens of a channel contiguous.
  __device__ __forceinline__ void store_bf16_cm(char* dst, int tid) const {
    static_assert(sizeof(Tin) == 2 && kL == 64, "bf16 rows of a 64-token chunk");
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = tid + i * NT, e = idx * kVec;
      if (idx >= kTot) break;
      const int t = e / D, r0 = e % D;
      const bf16x8v b = __builtin_bit_cast(bf16x8v, v[i]);
#pragma unroll
      for (int u = 0; u < kVec; ++u) *reinterpret_cast<__bf16*>(dst + sw8(r0 + u, t >> 3) + 2 * (t & 7)) = b[u];
    }
  }
};

// Row statistics of a chunk from its staged P1 and P2 rows: for each of the
// thread's loads (row t), sc1 = S_t / |p1_t| and sc2 = S_t / |p2_t|, the
// factors that turn the rows into S_t q_t and S_t k_t. A row's D / kVec loads
// sit in adjacent lanes, so each row takes a partial dot product per lane
// and a butterfly shuffle reduction that leaves the totals in every lane of
// the row; rows >= `rows` (loaded as zeros) get 0.
template <int NT, typename Tin, int D>
__device__ __forceinline__ void staged_row_stats(const Staged<NT, Tin, D>& g1, const Staged<NT, Tin, D>& g2, int rows,
                                                 float inv_scale, float (&sc1)[Staged<NT, Tin, D>::kN],
                                                 float (&sc2)[Staged<NT, Tin, D>::kN], int tid) {
  using St = Staged<NT, Tin, D>;
  constexpr int kLanes = D / St::kVec;              // lanes per row
  static_assert(kLanes <= 64 && 64 % kLanes == 0 && NT % 64 == 0, "a row's loads share a wave");
#pragma unroll
  for (int i = 0; i < St::kN; ++i) {
    const int idx = tid + i * NT;
    float x[St::kVec], y[St::kVec];
    g1.unpack(i, x);
    g2.unpack(i, y);
    float d12 = 0.0f, d11 = 0.0f, d22 = 0.0f;
#pragma unroll
    for (int u = 0; u < St::kVec; ++u) {
      d12 = fmaf(x[u], y[u], d12);
      d11 = fmaf(x[u], x[u], d11);
      d22 = fmaf(y[u], y[u], d22);
    }
#pragma unroll
    for (int w = kLanes / 2; w >= 1; w >>= 1) {
      d12 += __shfl_xor(d12, w, kLanes);
      d11 += __shfl_xor(d11, w, kLanes);
      d22 += __shfl_xor(d22, w, kLanes);
    }
    const int t = idx / kLanes;
    const float st = idx < St::kTot && t < rows ? sigmoid_f32(d12 * inv_scale) : 0.0f;
    // A zero row has no direction: its normalised coordinate is 0.
    sc1[i] = d11 > 0.0f ? st * (1.0f / sqrtf(d11)) : 0.0f;
    sc2[i] = d22 > 0.0f ? st * (1.0f / sqrtf(d22)) : 0.0f;
  }
}

// Runs mma(ks, op) for ks = 0 .. KS-1 with the LDS operands of each group of
// G k-steps fetched by load(ks, op) while the previous group's MFMAs run (the
// scheduling barriers keep the compiler from trading that overlap for
// registers). Fully unrolled: every index is a compile-time constant.
template <int KS, int G, typename Op, typename Load, typename Mma>
__device__ __forceinline__ void pipelined(Load load, Mma mma) {
  static_assert(KS % G == 0, "whole groups");
  constexpr int NG = KS / G;
  Op op[2][G];
#pragma unroll
  for (int u = 0; u < G; ++u) load(u, op[0][u]);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + 1 < NG) {
#pragma unroll
      for (int u = 0; u < G; ++u) load(G * (g + 1) + u, op[(g + 1) & 1][u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < G; ++u) mma(G * g + u, op[g & 1][u]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// In-place inclusive per-channel prefix of log2 alpha over the chunk (element
// (t, r) at b[t * rs + r * cs], holding alpha on entry; rows >= `rows` repeat
// the last value), so that e^{b_t - b_j} below is pow2 of a difference of
// these. alpha is clamped to [1e-30, 1] (NaN to 1e-30): log alpha
// stays finite, so differences of prefixes never form inf - inf, and a
// retention below 1e-30 already wipes the state within one step to fp32
// precision. NT / D threads share a channel, each a segment of consecutive
// tokens: every thread takes the logarithms of its segment and their running
// sum, then adds the totals of the earlier segments (in order). `tot` is NT
// floats of LDS scratch. Contains a barrier: every thread must call it.
template <int NT, int D>
__device__ __forceinline__ void decay_prefix(float* b, int rs, int cs, int rows, float* tot, int tid) {
  constexpr int kSeg = NT / D;
  constexpr int kLen = kL / kSeg;
  static_assert(NT % D == 0 && kL % kSeg == 0, "whole segments");
  const int r = tid % D, seg = tid / D, t0 = seg * kLen;
  float x[kLen];
#pragma unroll
  for (int i = 0; i < kLen; ++i) x[i] = b[(t0 + i) * rs + r * cs];
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kLen; ++i) {
    if (t0 + i < rows) acc += __builtin_amdgcn_logf(fminf(fmaxf(x[i], 1e-30f), 1.0f));
    x[i] = acc;
  }
  tot[seg * D + r] = acc;
  __syncthreads();
  float off = 0.0f;
  for (int q = 0; q < seg; ++q) off += tot[q * D + r];
#pragma unroll
  for (int i = 0; i < kLen; ++i) b[(t0 + i) * rs + r * cs] = x[i] + off;
}

// Phase 1: per (b*H + h, group of a.group consecutive chunks): the group's
// contribution to the state, dG = sum over its chunks c of
// Diag(e^{b_last of the later chunks of the group}) dC_c with
// dC_c = sum_j S_j (k_j o e^{b_last,c - b_j}) I_j^T, and the group's decay
// g = e^{sum of its b_last}, into the group's state slot. The chunks are
// taken in order with the state accumulators in registers: before chunk c is
// added, the accumulated rows are scaled by e^{b_last,c}. dC_c = Kt^T I is a
// d_h x d_h x 64 product: on v_mfma_f32_32x32x2_f32 for fp32 inputs, on
// v_mfma_f32_32x32x16_bf16 over Kt's split bf16 pair for bf16 inputs. The
// 32 x 32 state tiles are dealt to the 8 waves (tile w + 8 i to wave w, so a
// wave's tiles share one column block and its I operand, which comes
// straight from global memory into registers). P1 is only needed for the row
// statistics, which come from the staged registers; LDS holds Kt (then its
// split tiles) and the decay prefix, 66 KB at d_h = 128.
template <typename Tin, int D>
__global__ __launch_bounds__(kChunkThreads) void lin_chunk_kernel(LinArgs a, HeadParams hp) {
  constexpr int NT = kChunkThreads;
  constexpr bool kSplit = sizeof(Tin) == 2;           // bf16 MFMA on split operands
  __shared__ float kt[kL][D];     // S_j k_j, then S_j k_j e^{b_last - b_j}
  __shared__ float bt[kL][D];     // alpha_j, then b_j
  __shared__ float tot[NT];
  __shared__ __attribute__((aligned(16))) char itb[kSplit ? D * 128 : 16];   // bf16: I, channel-major
  const int nc = (a.T + kL - 1) / kL;
  const int ng = (nc + a.group - 1) / a.group;
  const int gi = blockIdx.x % ng;
  const int bh = blockIdx.x / ng;
  const int h = bh % a.H;
  const int c0 = gi * a.group, c1 = min(nc, c0 + a.group);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, lh = lane >> 5;
  constexpr int kW = NT / 64;
  constexpr int kT = D / 32;
  constexpr int kTiles = kT * kT;
  constexpr int kTPW = (kTiles + kW - 1) / kW;        // tiles per wave
  static_assert(kW % kT == 0, "a wave's tiles share their column block");
  const bool has_tiles = wave < kTiles;
  const int n = wave % kT;                            // the wave's column block
  char* const kh = reinterpret_cast<char*>(&kt[0][0]);
  char* const kl = kh + D * 128;

  // acc[i]: tile w + 8 i = (m, n), m = (w + 8 i) / kT; element r at row
  // 32 m + 8 (r >> 2) + 4 lh + (r & 3), column 32 n + l32.
  f32x16 acc[kTPW];
#pragma unroll
  for (int i = 0; i < kTPW; ++i) acc[i] = f32x16{};
  float bsum = 0.0f;                                  // thread r < D: sum of b_last,c[r]

  // A chunk's rows in registers, every load issued before any is used. bf16
  // inputs stage I like P1 and P2 (16-byte row loads), then store it as a
  // channel-major bf16 tile from which each MFMA's I operand is one 16-byte
  // read. fp32 inputs load the I operands of the wave's column block
  // directly, B[j][col] = I_j[col] with j = 2 ks + lh; rows past the chunk's
  // end read the last row (an address inside the tensor) and are zeroed
  // where they are used. With bf16 inputs the next chunk's rows are loaded
  // while the current one is computed: no register waits for them before the
  // next chunk. fp32 inputs (one chunk per group) load at the chunk's start.
  struct Rows {
    Staged<NT, Tin, D> g1, g2;
    Staged<NT, float, D> ga;
    Staged<NT, Tin, kSplit ? D : 8> gv;
    float bf[kSplit ? 1 : kL / 2];
  };
  auto fetch = [&](int c, Rows& f) __attribute__((always_inline)) {
    const int t0 = c * kL;
    const int rows = min(kL, a.T - t0);
    const size_t base = ((size_t)bh * a.T + t0) * D;
    const Tin* I = static_cast<const Tin*>(a.I) + base;
    if constexpr (kSplit) {
      f.gv.load(I, rows, threadIdx.x);
    } else if (has_tiles) {
#pragma unroll
      for (int ks = 0; ks < kL / 2; ++ks) f.bf[ks] = ld_val(I, (size_t)min(2 * ks + lh, rows - 1) * D + 32 * n + l32);
    }
    f.g1.load(static_cast<const Tin*>(a.P1) + base, rows, threadIdx.x);
    f.g2.load(static_cast<const Tin*>(a.P2) + base, rows, threadIdx.x);
    f.ga.load(a.alpha + base, rows, threadIdx.x);
  };

  Rows nx;
  if constexpr (kSplit) fetch(c0, nx);
  for (int c = c0; c < c1; ++c) {
    const int rows = min(kL, a.T - c * kL);
    if constexpr (!kSplit) {
      fetch(c, nx);           // the I operands are consumed in place: no load ahead
      if (has_tiles) {
#pragma unroll
        for (int ks = 0; ks < kL / 2; ++ks) nx.bf[ks] = 2 * ks + lh < rows ? nx.bf[ks] : 0.0f;
      }
    }
    {
      float sc1[Staged<NT, Tin, D>::kN], sc2[Staged<NT, Tin, D>::kN];
      staged_row_stats(nx.g1, nx.g2, rows, hp.scale * hp.inv_tau[h], sc1, sc2, threadIdx.x);
      // The row factors, for the output kernel: one lane per row writes them.
      constexpr int kLanes = D / Staged<NT, Tin, D>::kVec;
#pragma unroll
      for (int i = 0; i < Staged<NT, Tin, D>::kN; ++i) {
        const int idx = threadIdx.x + i * NT, t = idx / kLanes;
        if (idx < Staged<NT, Tin, D>::kTot && idx % kLanes == 0 && t < rows)
          *reinterpret_cast<float2*>(a.rowsc + ((size_t)bh * a.T + (size_t)c * kL + t) * 2) = make_float2(sc1[i], sc2[i]);
      }
      nx.g2.template store_scaled<false>(&kt[0][0], D, threadIdx.x, sc2);     // S_j k_j
      nx.ga.template store<false>(&bt[0][0], D, threadIdx.x);
      if constexpr (kSplit) nx.gv.store_bf16_cm(itb, threadIdx.x);
    }
    if constexpr (kSplit) {
      if (c + 1 < c1) fetch(c + 1, nx);
    }
    __syncthreads();
    decay_prefix<NT, D>(&bt[0][0], D, 1, rows, tot, threadIdx.x);
    __syncthreads();
    // Kt_j = S_j k_j o e^{b_last - b_j} (rows past the chunk's end: 0). The
    // bf16 path splits it into two channel-major bf16 tiles (channel r,
    // tokens contiguous) that take kt's place once every thread has read its
    // values.
    if constexpr (kSplit) {
      constexpr int kG = (kL * D / 8 + NT - 1) / NT;   // 8-token groups per thread
      float x[kG][8];
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        const int idx = threadIdx.x + k * NT, r = idx % D, cc = idx / D;
        if (idx >= kL * D / 8) break;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int t = 8 * cc + u;
          x[k][u] = t < rows ? kt[t][r] * pow2(bt[kL - 1][r] - bt[t][r]) : 0.0f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        const int idx = threadIdx.x + k * NT, r = idx % D, cc = idx / D;
        if (idx >= kL * D / 8) break;
        bf16x8v hi, lo;
        split_bf16(x[k], hi, lo);
        *reinterpret_cast<bf16x8v*>(kh + sw8(r, cc)) = hi;
        *reinterpret_cast<bf16x8v*>(kl + sw8(r, cc)) = lo;
      }
    } else {
      for (int e = threadIdx.x; e < kL * D; e += NT) {
        const int t = e / D, r = e % D;
        kt[t][r] = t < rows ? kt[t][r] * pow2(bt[kL - 1][r] - bt[t][r]) : 0.0f;
      }
    }
    __syncthreads();
    if (threadIdx.x < D) bsum += bt[kL - 1][threadIdx.x];
    if (has_tiles) {
      if (c > c0) {
        // The group's earlier chunks decay over this one.
#pragma unroll
        for (int i = 0; i < kTPW; ++i) {
          const int m = (wave + kW * i) / kT;
          if (m >= kT) break;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] *= pow2(bt[kL - 1][32 * m + 8 * (r >> 2) + 4 * lh + (r & 3)]);
        }
      }
      if constexpr (kSplit) {
        // A[r][j] = Kt_j[r] (hi and lo), B[j][col] = I_j[col], 16 tokens per
        // k-step; step st is the wave's tile st % kTPW at k-step st / kTPW.
        struct Op { bf16x8v h, l, b; };
        pipelined<kTPW * kL / 16, kTPW, Op>(
            [&](int st, Op& o) {
              const int m = (wave + kW * (st % kTPW)) / kT, kk = st / kTPW;
              o.h = lds_bf16x8(kh, sw8(32 * m + l32, 2 * kk + lh));
              o.l = lds_bf16x8(kl, sw8(32 * m + l32, 2 * kk + lh));
              o.b = lds_bf16x8(itb, sw8(32 * n + l32, 2 * kk + lh));
            },
            [&](int st, const Op& o) {
              const int i = st % kTPW;
              acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.h, o.b, acc[i], 0, 0, 0);
              acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.l, o.b, acc[i], 0, 0, 0);
            });
      } else {
        struct Op { float a[kTPW]; };
        pipelined<kL / 2, 4, Op>(
            [&](int ks, Op& o) {
#pragma unroll
              for (int i = 0; i < kTPW; ++i) o.a[i] = kt[2 * ks + lh][32 * ((wave + kW * i) / kT) + l32];
            },
            [&](int ks, const Op& o) {
#pragma unroll
              for (int i = 0; i < kTPW; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(o.a[i], nx.bf[ks], acc[i], 0, 0, 0);
            });
      }
    }
    __syncthreads();                                  // kt and bt are rewritten by the next chunk
  }
  if (has_tiles) {
    float* dG = a.state + ((size_t)bh * ng + gi) * (size_t)D * D;
#pragma unroll
    for (int i = 0; i < kTPW; ++i) {
      const int m = (wave + kW * i) / kT;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dG[(size_t)(32 * m + 8 * (r >> 2) + 4 * lh + (r & 3)) * D + 32 * n + l32] = acc[i][r];
    }
  }
  if (threadIdx.x < D) a.decay[((size_t)bh * ng + gi) * D + threadIdx.x] = pow2(bsum);
}

// Phase 2: per state element (b*H + h, r, col), over the groups of chunks:
// Cin_0 = 0, Cin_{g+1} = e^{sum of the group's b_last}[r] Cin_g + dG_g; each
// group slot is overwritten with the state entering the group's first chunk,
// and the final state goes to a.final (if given).
// A thread owns 4 consecutive elements of one row r (16-byte accesses; the
// state buffers are 16-byte aligned) and loads the contributions and decays
// of kScanAhead groups before it uses them, so that many loads are in flight
// per thread.
constexpr int kScanAhead = 8;

template <int D>
__global__ __launch_bounds__(kScanThreads) void lin_scan_kernel(LinArgs a) {
  constexpr int kQ = D * D / 4;                 // 4-element groups per state
  const long long idx = (long long)blockIdx.x * kScanThreads + threadIdx.x;
  if (idx >= (long long)a.B * a.H * kQ) return;
  const int e = 4 * (int)(idx % kQ);
  const long long bh = idx / kQ;
  const int r = e / D;
  const int nc = (a.T + kL - 1) / kL;
  const int ng = (nc + a.group - 1) / a.group;
  float4* st = reinterpret_cast<float4*>(a.state + (size_t)bh * ng * D * D + e);
  const float* g = a.decay + (size_t)bh * ng * D + r;
  float4 C = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto step = [&](float4& slot, float4 dc, float gc) __attribute__((always_inline)) {
    slot = C;
    C = make_float4(fmaf(gc, C.x, dc.x), fmaf(gc, C.y, dc.y), fmaf(gc, C.z, dc.z), fmaf(gc, C.w, dc.w));
  };
  int c = 0;
  for (; c + kScanAhead <= ng; c += kScanAhead) {
    float4 dc[kScanAhead];
    float gc[kScanAhead];
#pragma unroll
    for (int k = 0; k < kScanAhead; ++k) {
      dc[k] = st[(size_t)(c + k) * kQ];
      gc[k] = g[(size_t)(c + k) * D];
    }
#pragma unroll
    for (int k = 0; k < kScanAhead; ++k) step(st[(size_t)(c + k) * kQ], dc[k], gc[k]);
  }
  for (; c < ng; ++c) step(st[(size_t)c * kQ], st[(size_t)c * kQ], g[(size_t)c * D]);
  if (a.final) *reinterpret_cast<float4*>(a.final + (size_t)bh * D * D + e) = C;
}

// Phase 3: per (b*H + h, chunk): Y = I + at I + Qt Cin, with
//   at[t][j] = S_t S_j sum_r q_{t,r} k_{j,r} e^{b_{t,r} - b_{j,r}}  (j < t),
//   Qt[t][r] = S_t q_{t,r} e^{b_{t,r}}.
// at is built per 16-row sub-block pair on v_mfma_f32_16x16x4_f32, the decay
// factored through a reference row R as e^{b_t - b_R} e^{b_R - b_j}: off the
// diagonal (tb > jb) R = 16 jb + 15 (j <= R < t, both exponents <= 0); on the
// diagonal R is the block's middle row, which keeps every exponent within
// +-40 unless the retention falls by more than e^-40 within 8 tokens on some
// channel; such a block takes the exact per-element exponentials instead.
// The output is one accumulation over j (at I) and r (Qt Cin) per 32 x 32
// tile, one tile per wave, with its column of Cin in registers: on
// v_mfma_f32_32x32x2_f32 for fp32 inputs; for bf16 inputs on
// v_mfma_f32_32x32x16_bf16 with at, Qt and Cin split into bf16 pairs (I is
// exact), from XOR-swizzled bf16 tiles. The fp32 LDS arrays are stored
// channel-major ([r][t], rows padded to 65 floats) so that the operand reads
// and transposing writes are conflict-free.
// Persistent: a work-group takes chunks blockIdx.x + k gridDim.x, and the
// next chunk's rows are loaded into registers while the current one is
// computed (its Cin column, needed last, is loaded at the iteration's start).
template <typename Tin, int D>
struct OutPrefetch {
  Staged<kOutThreads, Tin, D> p1, p2, in;
  Staged<kOutThreads, float, D> al;
  float2 sc[Staged<kOutThreads, Tin, D>::kN];    // the row factors of the p1 / p2 loads' rows
};

template <typename Tin, int D>
__global__ __launch_bounds__(kOutThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void lin_out_kernel(LinArgs a, HeadParams hp) {
  constexpr int NT = kOutThreads;
  constexpr int kW = NT / 64;
  constexpr int kP = kL + 1;      // padded row length of the channel-major arrays
  __shared__ float qT[D][kP];     // S_t q_{t,r}, then S_t q_{t,r} e^{b_{t,r}}
  __shared__ float kT[D][kP];     // S_j k_{j,r}
  __shared__ float bT[D][kP];     // b_{t,r}
  __shared__ float it[kL][D];     // I_j
  __shared__ float atT[kL][kP];   // at[t][j] stored as atT[j][t] (the prefix's scratch before)
  static_assert(kL * kP >= NT, "prefix scratch fits in atT");
  // bf16 inputs: I is kept as a channel-major bf16 tile in the memory of
  // `it`, at as split bf16 tiles (token-major) in that of atT; once the
  // sub-block tasks are done, Qt goes as split bf16 tiles (token-major) into
  // the memory of qT and Kt_j = S_j k_j o e^{b_last - b_j} (the operand of the
  // state update) as split bf16 tiles (channel-major) into that of kT.
  constexpr bool kSplit = sizeof(Tin) == 2;
  char* const itb = reinterpret_cast<char*>(&it[0][0]);
  char* const ath = reinterpret_cast<char*>(&atT[0][0]);
  char* const atl = ath + kL * 128;
  char* const qth = reinterpret_cast<char*>(&qT[0][0]);
  char* const qtl = qth + kL * 2 * D;
  char* const kth = reinterpret_cast<char*>(&kT[0][0]);
  char* const ktl = kth + D * 128;
  static_assert(2 * kL * 128 <= (int)sizeof(atT) && 4 * kL * D <= (int)sizeof(qT) && 4 * kL * D <= (int)sizeof(kT),
                "split tiles fit");
  // at[t][j] into its tile(s).
  auto put_at = [&](int t, int j, float v) __attribute__((always_inline)) {
    if constexpr (kSplit) {
      const __bf16 hi = (__bf16)v;
      const int off = sw8(t, j >> 3) + 2 * (j & 7);
      *reinterpret_cast<__bf16*>(ath + off) = hi;
      *reinterpret_cast<__bf16*>(atl + off) = (__bf16)(v - (float)hi);
    } else {
      atT[j][t] = v;
    }
  };
  const int nc = (a.T + kL - 1) / kL;
  const int ng = (nc + a.group - 1) / a.group;
  const int total_g = a.B * a.H * ng;
  constexpr int kTN = D / 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool has_tile = wave < 2 * kTN;              // output tile (m, n) of this wave
  const int n_out = wave % kTN, m_out = wave / kTN;
  // Lane-dependent indices are re-formed from an opaque copy of threadIdx.x
  // in every iteration of the chunk loop: otherwise the compiler hoists every
  // unrolled LDS address out of the loop and runs out of registers.
  int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;

  // Loads of chunk g's rows (global index g = bh * nc + c) into registers.
  auto fetch = [&](int g, OutPrefetch<Tin, D>& f) __attribute__((always_inline)) {
    const int c = g % nc, bh = g / nc;
    const int rows = min(kL, a.T - c * kL);
    const size_t base = ((size_t)bh * a.T + (size_t)c * kL) * D;
    f.p1.load(static_cast<const Tin*>(a.P1) + base, rows, tid);
    f.p2.load(static_cast<const Tin*>(a.P2) + base, rows, tid);
    f.in.load(static_cast<const Tin*>(a.I) + base, rows, tid);
    f.al.load(a.alpha + base, rows, tid);
    constexpr int kLanes = D / Staged<NT, Tin, D>::kVec;
#pragma unroll
    for (int i = 0; i < Staged<NT, Tin, D>::kN; ++i) {
      const int idx = tid + i * NT, t = idx / kLanes;
      f.sc[i] = idx < Staged<NT, Tin, D>::kTot && t < rows
                    ? *reinterpret_cast<const float2*>(a.rowsc + ((size_t)bh * a.T + (size_t)c * kL + t) * 2)
                    : make_float2(0.0f, 0.0f);
    }
  };

  // The work-group takes the groups gl = blockIdx.x + k gridDim.x (gl = bh ng
  // + group within the head) and walks each group's chunks in order, with
  // the entering state of the current chunk in registers: loaded at the
  // group's first chunk, stepped on chip to the next one (bf16 inputs; fp32
  // inputs come with one chunk per group).
  auto chunk_of = [&](int gl, int k) { return (gl / ng) * nc + (gl % ng) * a.group + k; };
  // cf: this wave's column of Cin, element ks at cf[ks / 16][ks % 16]. fp32:
  // B[r][col] with r = 2 ks + lh; bf16: the order of an MFMA accumulator,
  // state row 32 (ks / 16) + 8 ((ks / 4) % 4) + 4 lh + ks % 4, so that the
  // update accumulates into it.
  f32x16 cf[kTN];
  OutPrefetch<Tin, D> nx;
  if ((int)blockIdx.x < total_g) fetch(chunk_of(blockIdx.x, 0), nx);
  for (int gl = blockIdx.x, k = 0; gl < total_g;) {
    tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    l32 = lane & 31;
    lh = lane >> 5;
    const int len = min(a.group, nc - (gl % ng) * a.group);
    const int g = chunk_of(gl, k);
    const int ngl = k + 1 < len ? gl : gl + (int)gridDim.x, nk = k + 1 < len ? k + 1 : 0;
    const int c = g % nc, bh = g / nc;
    const int rows = min(kL, a.T - c * kL);
    Tin* Y = static_cast<Tin*>(a.Y) + ((size_t)bh * a.T + (size_t)c * kL) * D;
    // The previous chunk's LDS is free (the barrier that ends its iteration).
    {
      // The row factors S_t / |p1_t| and S_t / |p2_t| that the chunk kernel wrote.
      float sc1[Staged<NT, Tin, D>::kN], sc2[Staged<NT, Tin, D>::kN];
#pragma unroll
      for (int i = 0; i < Staged<NT, Tin, D>::kN; ++i) {
        sc1[i] = nx.sc[i].x;
        sc2[i] = nx.sc[i].y;
      }
      nx.p1.template store_scaled<true>(&qT[0][0], kP, tid, sc1);    // S_t q_t
      nx.p2.template store_scaled<true>(&kT[0][0], kP, tid, sc2);    // S_j k_j
    }
    if constexpr (kSplit) nx.in.store_bf16_cm(itb, tid);
    else nx.in.template store<false>(&it[0][0], D, tid);
    nx.al.template store<true>(&bT[0][0], kP, tid);
    if (has_tile && k == 0) {
      const float* cin = a.state + (size_t)gl * D * D;
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks) {
        const int r = kSplit ? 32 * (ks >> 4) + 8 * ((ks >> 2) & 3) + 4 * lh + (ks & 3) : 2 * ks + lh;
        cf[ks >> 4][ks & 15] = cin[(size_t)r * D + 32 * n_out + l32];
      }
    }
    if (ngl < total_g) fetch(chunk_of(ngl, nk), nx);
    __syncthreads();
    decay_prefix<NT, D>(&bT[0][0], 1, kP, rows, &atT[0][0], tid);
    __syncthreads();

    // Sub-block tasks on the 8 waves. The pairs below the diagonal (tb, jb),
    // tb > jb, factor through R = 16 jb + 15: waves 0 and 1 take two pairs
    // that share jb, (1,0) + (2,0) and (2,1) + (3,1), with one key-side
    // operand and two accumulators; waves 2-5 take the diagonal blocks; waves
    // 6 and 7 the pairs (3,0) and (3,2).
    static_assert(kW == 8, "the task assignment is for 8 waves");
    {
      const int l16 = lane & 15, lq = lane >> 4;
      auto pairs = [&](auto nt, int tb0, int tb1, int jb) __attribute__((always_inline)) {
        constexpr int N = decltype(nt)::value;
        const int R = 16 * jb + 15, j = 16 * jb + l16;
        const int tq[2] = {16 * tb0 + l16, 16 * tb1 + l16};
        f32x4 acc[N];
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n] = f32x4{};
        if constexpr (kSplit) {
          // On v_mfma_f32_16x16x32_bf16 over split operands: k-group kk
          // takes channels r = 32 kk + 8 lq + u (u = 0..7) in two steps of
          // four.
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            const int r0 = 32 * kk + 8 * lq;
            float ref[8], x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              ref[u] = bT[r0 + u][R];
              x[u] = kT[r0 + u][j] * pow2(ref[u] - bT[r0 + u][j]);
            }
            bf16x8v bh, bl;
            split_bf16(x, bh, bl);
#pragma unroll
            for (int n = 0; n < N; ++n) {
#pragma unroll
              for (int u = 0; u < 8; ++u) x[u] = qT[r0 + u][tq[n]] * pow2(bT[r0 + u][tq[n]] - ref[u]);
              bf16x8v ah, al;
              split_bf16(x, ah, al);
              acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[n], 0, 0, 0);
              acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[n], 0, 0, 0);
              acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[n], 0, 0, 0);
            }
          }
        } else {
        struct OpP { float ref, k, bk, q[N], bq[N]; };
        pipelined<D / 4, 8 / N, OpP>(
            [&](int ks, OpP& o) {
              const int r = 4 * ks + lq;
              o.ref = bT[r][R];
              o.k = kT[r][j];
              o.bk = bT[r][j];
#pragma unroll
              for (int n = 0; n < N; ++n) {
                o.q[n] = qT[r][tq[n]];
                o.bq[n] = bT[r][tq[n]];
              }
            },
            [&](int ks, const OpP& o) {
              const float bv = o.k * pow2(o.ref - o.bk);
#pragma unroll
              for (int n = 0; n < N; ++n)
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.q[n] * pow2(o.bq[n] - o.ref), bv, acc[n], 0, 0, 0);
            });
        }
        // acc[n][i]: row t = 16 tb + 4 lq + i, column j = 16 jb + l16.
#pragma unroll
        for (int n = 0; n < N; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) put_at(16 * (n ? tb1 : tb0) + 4 * lq + i, 16 * jb + l16, acc[n][i]);
      };
      if (wave < 2) {
        pairs(std::integral_constant<int, 2>{}, wave + 1, wave + 2, wave);
      } else if (wave >= 6) {
        pairs(std::integral_constant<int, 1>{}, 3, 3, wave == 6 ? 0 : 2);
      } else {
        const int tb = wave - 2;
        const int R = 16 * tb + 7;
        // b is non-increasing in t, so the extreme exponents are those of
        // the block's first and last rows.
        int ok = 1;
        for (int r = lane; r < D; r += 64) {
          const float br = bT[r][R];
          ok &= (bT[r][16 * tb] - br <= kFactorBound) & (br - bT[r][16 * tb + 15] <= kFactorBound);
        }
        if (__all(ok)) {
          const int t = 16 * tb + l16, j = 16 * tb + l16;
          f32x4 acc = {};
          if constexpr (kSplit) {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
              const int r0 = 32 * kk + 8 * lq;
              float av[8], bv[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const float ref = bT[r0 + u][R];
                av[u] = qT[r0 + u][t] * pow2(bT[r0 + u][t] - ref);
                bv[u] = kT[r0 + u][j] * pow2(ref - bT[r0 + u][j]);
              }
              bf16x8v ah, al, bh, bl;
              split_bf16(av, ah, al);
              split_bf16(bv, bh, bl);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
            }
          } else {
          struct OpAt { float ref, q, bq, k, bk; };
          pipelined<D / 4, 8, OpAt>(
              [&](int ks, OpAt& o) {
                const int r = 4 * ks + lq;
                o.ref = bT[r][R];
                o.q = qT[r][t];
                o.bq = bT[r][t];
                o.k = kT[r][j];
                o.bk = bT[r][j];
              },
              [&](int ks, const OpAt& o) {
                const float av = o.q * pow2(o.bq - o.ref);
                const float bv = o.k * pow2(o.ref - o.bk);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
              });
          }
          // acc[i]: row t = 16 tb + 4 lq + i, column j = 16 tb + l16; only
          // j < t is history.
#pragma unroll
          for (int i = 0; i < 4; ++i) put_at(16 * tb + 4 * lq + i, 16 * tb + l16, l16 < 4 * lq + i ? acc[i] : 0.0f);
        } else {
          for (int e = lane; e < 256; e += 64) {
            const int tl = e >> 4, jl = e & 15;
            const int t = 16 * tb + tl, j = 16 * tb + jl;
            float acc = 0.0f;
            if (jl < tl) {
              for (int r = 0; r < D; ++r) acc = fmaf(qT[r][t] * kT[r][j], pow2(bT[r][t] - bT[r][j]), acc);
            }
            put_at(t, j, acc);
          }
        }
      }
    }
    // The zero blocks above the diagonal.
    // Block p of (0,1) (0,2) (0,3) (1,2) (1,3) (2,3), found by arithmetic:
    // an indexed table would sit in constant memory and its load's wait
    // would also drain the column and prefetch loads still in flight.
    for (int e = tid; e < 6 * 256; e += NT) {
      const int p = e >> 8, tl = (e >> 4) & 15, jl = e & 15;
      const int tb = (p >= 3) + (p >= 5);
      const int jb = p + 1 - 2 * (p >= 3) - (p >= 5);
      put_at(16 * tb + tl, 16 * jb + jl, 0.0f);
    }
    __syncthreads();
    // Qt = S q o e^{b} (every exponent <= 0): in place, or split into
    // token-major bf16 tiles over qT, whose 16-byte chunk cc holds channels
    // 16 (cc / 2) + 4 (cc % 2) + 8 (u / 4) + u % 4 (u = 0..7), the state rows
    // that the lanes of half cc % 2 hold in cf. The bf16 path also splits
    // Kt = S k o e^{b_last - b} into channel-major tiles over kT. Both read
    // every value first: the tiles overwrite the arrays they are formed from.
    if constexpr (kSplit) {
      constexpr int kG = (kL * D / 8 + NT - 1) / NT;
      float xq[kG][8], xk[kG][8];
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        const int e = tid + q * NT;
        if (e >= kL * D / 8) break;
        const int t = e % kL, cc = e / kL;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = 16 * (cc >> 1) + 4 * (cc & 1) + 8 * (u >> 2) + (u & 3);
          xq[q][u] = qT[r][t] * pow2(bT[r][t]);
        }
        const int rk = e % D, ck = e / D;
#pragma unroll
        for (int u = 0; u < 8; ++u) xk[q][u] = kT[rk][8 * ck + u] * pow2(bT[rk][kL - 1] - bT[rk][8 * ck + u]);
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kG; ++q) {
        const int e = tid + q * NT;
        if (e >= kL * D / 8) break;
        const int t = e % kL, cc = e / kL, rk = e % D, ck = e / D;
        bf16x8v hi, lo;
        split_bf16(xq[q], hi, lo);
        *reinterpret_cast<bf16x8v*>(qth + swd<D>(t, cc)) = hi;
        *reinterpret_cast<bf16x8v*>(qtl + swd<D>(t, cc)) = lo;
        split_bf16(xk[q], hi, lo);
        *reinterpret_cast<bf16x8v*>(kth + sw8(rk, ck)) = hi;
        *reinterpret_cast<bf16x8v*>(ktl + sw8(rk, ck)) = lo;
      }
    } else {
      for (int e = tid; e < kL * D; e += NT) {
        const int r = e / kL, t = e % kL;
        qT[r][t] *= pow2(bT[r][t]);
      }
    }
    __syncthreads();

    // Y tile (m, n): rows 32 m .., columns 32 n ...
    if (has_tile) {
      const int col = 32 * n_out + l32, t = 32 * m_out + l32;
      f32x16 acc = {};
      if constexpr (kSplit) {
        // at I: A = at (hi, lo), B = I (exact); Qt Cin: A = Qt (hi, lo), B = Cin
        // (hi, lo, split here); 16 tokens or channels per k-step.
        struct OpA { bf16x8v h, l, b; };
        pipelined<kL / 16, 2, OpA>(
            [&](int kk, OpA& o) {
              o.h = lds_bf16x8(ath, sw8(t, 2 * kk + lh));
              o.l = lds_bf16x8(atl, sw8(t, 2 * kk + lh));
              o.b = lds_bf16x8(itb, sw8(col, 2 * kk + lh));
            },
            [&](int kk, const OpA& o) {
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.h, o.b, acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.l, o.b, acc, 0, 0, 0);
            });
        struct OpQ { bf16x8v h, l; };
        pipelined<D / 16, 2, OpQ>(
            [&](int kk, OpQ& o) {
              o.h = lds_bf16x8(qth, swd<D>(t, 2 * kk + lh));
              o.l = lds_bf16x8(qtl, swd<D>(t, 2 * kk + lh));
            },
            [&](int kk, const OpQ& o) {
              float x[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = cf[kk >> 1][8 * (kk & 1) + e];
              bf16x8v ch, cl;
              split_bf16(x, ch, cl);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.h, ch, acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.h, cl, acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.l, ch, acc, 0, 0, 0);
            });
      } else {
        struct Op2 { float a, b; };
        pipelined<kL / 2, 8, Op2>(
            [&](int ks, Op2& o) {
              o.a = atT[2 * ks + lh][t];
              o.b = it[2 * ks + lh][col];
            },
            [&](int ks, const Op2& o) { acc = __builtin_amdgcn_mfma_f32_32x32x2f32(o.a, o.b, acc, 0, 0, 0); });
        pipelined<D / 2, 8, float>([&](int ks, float& o) { o = qT[2 * ks + lh][t]; },
                                   [&](int ks, float o) { acc = __builtin_amdgcn_mfma_f32_32x32x2f32(o, cf[ks >> 4][ks & 15], acc, 0, 0, 0); });
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = 32 * m_out + 8 * (r >> 2) + 4 * lh + (r & 3);
        float iv;
        if constexpr (kSplit) iv = (float)*reinterpret_cast<const __bf16*>(itb + sw8(col, tr >> 3) + 2 * (tr & 7));
        else iv = it[tr][col];
        if (tr < rows) Y[(size_t)tr * D + col] = from_f32<Tin>(iv + acc[r]);
      }
      if constexpr (kSplit) {
        if (k + 1 < len) {
          // The next chunk's entering state: cf = e^{b_last} cf + (Kt^T I)
          // column, accumulated into cf on the same split operands (the
          // chunk is whole).
#pragma unroll
          for (int ks = 0; ks < D / 2; ++ks)
            cf[ks >> 4][ks & 15] *= pow2(bT[32 * (ks >> 4) + 8 * ((ks >> 2) & 3) + 4 * lh + (ks & 3)][kL - 1]);
          struct OpU { bf16x8v h, l, b; };
          pipelined<kTN * kL / 16, 2, OpU>(
              [&](int st, OpU& o) {
                const int m = st / (kL / 16), kk = st % (kL / 16);
                o.h = lds_bf16x8(kth, sw8(32 * m + l32, 2 * kk + lh));
                o.l = lds_bf16x8(ktl, sw8(32 * m + l32, 2 * kk + lh));
                o.b = lds_bf16x8(itb, sw8(col, 2 * kk + lh));
              },
              [&](int st, const OpU& o) {
                const int m = st / (kL / 16);
                cf[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.h, o.b, cf[m], 0, 0, 0);
                cf[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.l, o.b, cf[m], 0, 0, 0);
              });
        }
      }
    }
    __syncthreads();
    gl = ngl;
    k = nk;
  }
}

// Chunks per group: the largest power of two up to kMaxGroup that still
// leaves kMinGroupsPerCu groups per compute unit (1 if none does). Larger
// groups move fewer states through HBM (one per group is written, scanned
// and read back) but walk more chunks in sequence per work-group. fp32 inputs
// take one chunk per group (their output kernel has no on-chip update).
constexpr int kMaxGroup = 16;
constexpr int kMinGroupsPerCu = 1;

template <typename Tin, int D>
hipError_t launch_typed(const LinArgs& args, const HeadParams& hp, hipStream_t s) {
  const int nc = (args.T + kL - 1) / kL;
  const long long chunks = (long long)args.B * args.H * nc;
  const long long scan_threads = (long long)args.B * args.H * D * D / 4;
  if (chunks > 0x7fffffffLL || (scan_threads + kScanThreads - 1) / kScanThreads > 0x7fffffffLL) return hipErrorInvalidValue;
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  LinArgs a = args;
  a.group = 1;
  if (sizeof(Tin) == 2) {
    for (int gsz = kMaxGroup; gsz > 1; gsz >>= 1) {
      if ((long long)args.B * args.H * ((nc + gsz - 1) / gsz) >= (long long)kMinGroupsPerCu * n_cu) {
        a.group = gsz;
        break;
      }
    }
  }
  const long long groups = (long long)args.B * args.H * ((nc + a.group - 1) / a.group);
  hipLaunchKernelGGL((lin_chunk_kernel<Tin, D>), dim3((unsigned)groups), dim3(kChunkThreads), 0, s, a, hp);
  hipLaunchKernelGGL((lin_scan_kernel<D>), dim3((unsigned)((scan_threads + kScanThreads - 1) / kScanThreads)),
                     dim3(kScanThreads), 0, s, a);
  // The output kernel is persistent: one work-group per compute unit (its LDS
  // admits one).
  hipLaunchKernelGGL((lin_out_kernel<Tin, D>), dim3((unsigned)(groups < n_cu ? groups : n_cu)), dim3(kOutThreads), 0, s,
                     a, hp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinArgs& a, const HeadParams& hp, bool bf16, hipStream_t s) {
  switch (a.d_h) {
    case 32: return bf16 ? launch_typed<__bf16, 32>(a, hp, s) : launch_typed<float, 32>(a, hp, s);
    case 64: return bf16 ? launch_typed<__bf16, 64>(a, hp, s) : launch_typed<float, 64>(a, hp, s);
    case 128: return bf16 ? launch_typed<__bf16, 128>(a, hp, s) : launch_typed<float, 128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

// bf16 MFMA backward of the causal Self-Exchange Relation for gfx950
// ("Ask Self, Ask Others: Relation Is All You Need", Eq. (1)-(3); the
// FlashRelation backward of App. A.3 recomputes the evidence per tile from the
// stored per-row log normaliser instead of keeping U, R or F).
//
// Two kernels share the tile machinery of the forward (mfma_tile.h); both
// recompute the Exchange evidence u = p1_i . p2_j / sqrt(d_h) and
// g = dY_i . V_j per tile and form, for j < i,
//   F_ij = 2^(SiLU(u) log2 e - L2_i),  L2_i = (LSE_i + lambda log i) log2 e,
//   W_ij = F_ij (g - D_i) SiLU'(u)      (= dU_ij; SiLU'(u) = s (1 + u (1 - s)))
// with the row statistics L2_i and D_i = dY_i . Y_i (the G accumulators start
// at -D_i, so the MFMA yields g - D_i directly).
//
// dq (query gradient): 8 waves x 32 query rows, key tiles of 64 rows; per tile
//   U^T[key][q] = P2 . P1^T and G^T[key][q] = V . dY^T (evidence; P1 and dY
//   rows of the wave's queries in registers), then
//   dP1^T[d][q] += P2^T[d][key] W^T[key][q] (transport).
//   LDS per key tile: P2 in the row layout and the transposed layout, V in
//   the row layout; a ring of 3 tiles, one barrier per tile. dq runs first:
//   its prologue forms the row statistics of its rows (stored per 64-row
//   tile) and its epilogue the chunk's (dtau, dlambda) partial.
// dkv (key/value gradients): 16 keys per wave, query tiles of 64 rows; per
//   16-query block U[q][key] = P1 . P2^T and G[q][key] = dY . V^T (P2 and V
//   rows of the wave's keys in registers), F and W, then
//   dV^T[d][key] += dY^T[d][q] F[q][key] and dP2^T[d][key] += P1^T[d][q] W[q][key]
//   on v_mfma_f32_16x16x32_bf16, both accumulators in the wave. LDS per query
//   tile: P1 and dY in one row layout plus the tile's row statistics; a ring
//   of 4 tiles, one barrier per pair of tiles.
// The Self entries (diagonal) enter in the epilogues from the row
// statistics: dP1_i += dU_ii p2_i / sqrt(d_h), dP2_j += dU_jj p1_j / sqrt(d_h),
// dV_j += F_jj dY_j.
#include <type_traits>

#include "mfma_tile.h"
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

using namespace mfma;

constexpr int kDqWaves = 8;
constexpr int kDqThreads = kDqWaves * 64;
constexpr int kDqRows = kDqWaves * 32;     // query rows per dq work-group
constexpr int kDqSlots = 3;
static_assert(kDqRows == kPrepRows, "a dq work-group's rows are one (dtau, dlambda) partial chunk");

template <int D>
struct DqCfg : TileLayout<D> {
  using L = TileLayout<D>;
  // Slot: [P2 row layout][V row layout][P2 transposed layout].
  static constexpr int kSlotBytes = 2 * L::kKBytes + L::kVBytes;
  static constexpr int kLdsBytes = kDqSlots * kSlotBytes;
  static constexpr int kPer = L::kBlocks / kDqWaves;    // blocks per wave, tile and layout
  static constexpr int kDmaTile = 3 * kPer;              // direct loads per wave and tile
  static_assert(L::kBlocks % kDqWaves == 0, "each wave moves whole blocks");
};


// Mode of a 32-row block of the scanned operand for a wave whose own 32-row
// block is `own`: 0 = no pair (i, j) with j < i, 1 = all pairs, 2 = diagonal
// block (masked inside).
__device__ __forceinline__ int mode_keys_below(int blk, int own) { return blk < own ? 1 : (blk == own ? 2 : 0); }
__device__ __forceinline__ int mode_queries_above(int blk, int own) { return blk > own ? 1 : (blk == own ? 2 : 0); }

__device__ __forceinline__ int64_t stat_at(int64_t bh, int nt, int r, int k) {
  return ((bh * nt + r / kStatRows) * 4 + k) * kStatRows + (r % kStatRows);
}

// Weight terms of one raw evidence value x = p1 . p2 (k2 = log2 e / sqrt(d_h),
// c = 1 / sqrt(d_h), L2 = the row's (LSE + lambda log i) log2 e):
//   s = sigmoid(u), u = x c;  F = 2^(u s log2 e - L2);  SiLU'(u) = s + u (s - s^2).
struct Terms {
  float F, dsilu;
  __device__ __forceinline__ Terms(float x, float k2, float c, float L2) {
    const float a2 = x * k2;
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a2));
    F = __builtin_amdgcn_exp2f(fmaf(a2, sg, -L2));
    dsilu = fmaf(x * c, fmaf(-sg, sg, sg), sg);
  }
};

// dq weights of one 32-key block: W^T[key][q] for this lane's query (row lq),
// register r <-> key 8 (r / 4) + 4 hf + r % 4 of the block; gm holds
// dY_q . V_key - D_q.
__device__ __forceinline__ void dq_weights(const f32x16& s, const f32x16& gm, float k2, float c, float L2,
                                           bool diag, int hf, int lq, u32x4 (&pw)[2]) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    float w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const Terms t(s[r + e], k2, c, L2);
      float v = t.F * gm[r + e] * t.dsilu;
      if (diag) v = (8 * ((r + e) >> 2) + 4 * hf + ((r + e) & 3)) < lq ? v : 0.0f;
      w[e] = v;
    }
    pw[r >> 3][(r & 7) >> 1] = pack_bf16(w[0], w[1]);
  }
}

// Store 4 consecutive bf16 of a row (8 bytes).
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16(a, b), pack_bf16(c, d)};
}
__device__ __forceinline__ void load4(const __bf16* p, float (&x)[4]) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
}

template <bool B>
using Tag = std::integral_constant<bool, B>;

// D: head size of the tile layout (64 or 128); DR: the rows' real head size
// (32 and 48 run on the 64 layout, 80 on the 128 one, with zero-filled pad chunks, as in
// the forward: exact evidence, zero pad rows of the transports, pad columns
// not stored).
template <int D, int DR = D>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_kernel(BwdArgs a, HeadParams hp) {
  static_assert(DR % 16 == 0 && DR <= D && DR >= 32, "real head size within the layout");
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];

  const int T = a.T;
  const int nq = (T + kDqRows - 1) / kDqRows;
  const int BH = a.B * a.H;
  const int qt = nq - 1 - (int)blockIdx.x / BH;       // longest histories first
  const int bh = (int)blockIdx.x % BH;
  const int nt = (T + kStatRows - 1) / kStatRows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;

  const size_t head = (size_t)bh * (size_t)T * DR;
  const long long head_bytes = (long long)T * DR * 2;
  const __bf16* P1 = static_cast<const __bf16*>(a.P1) + head;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  const __bf16* dY = static_cast<const __bf16*>(a.dY) + head;
  __bf16* dP1 = static_cast<__bf16*>(a.dP1) + head;

  const int q0 = qt * kDqRows;
  const int qrow = q0 + wave * 32 + lq;               // may be >= T: loads give 0, stores drop
  const int own = q0 / 32 + wave;                     // the wave's 32-row block

  // Rows of P1 and dY as evidence B operands: lane holds row qrow, columns
  // 16 ds + 8 hf + 0..7.
  bf16x8 qf[C::kDs], yf[C::kDs];
  {
    const auto rP1 = rsrc(P1, head_bytes);
    const auto rdY = rsrc(dY, head_bytes);
    const int qoff = qrow * (DR * 2) + hf * 16;
#pragma unroll
    for (int ds = 0; ds < C::kDs; ++ds) {
      const int o = ds < DR / 16 ? qoff + ds * 32 : kOutOfRange;   // pad k-steps read 0
      qf[ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP1, o, 0, 0));
      yf[ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdY, o, 0, 0));
    }
  }
  // Row statistics of this work-group's rows, from the rows of P1, P2, V, Y
  // and dY (each lane takes the dot products over its half of the columns):
  //   L2_i = (LSE_i + lambda log i) log2 e,  D_i = dY_i . Y_i,
  //   F_ii = e^{S_i - LSE_i},  dU_ii / sqrt(d_h) = F_ii (dY_i . V_i - D_i) S_i (1 - S_i) / (tau sqrt(d_h)),
  // stored per 64-row tile for the key/value kernel (launched after this
  // one), and this 256-row chunk's (dtau, dlambda) partial.
  const bool valid = qrow < T;
  float L2 = INFINITY, negD = 0.0f, us = 0.0f, ptau = 0.0f, plam = 0.0f;
  {
    const auto rY = rsrc(static_cast<const __bf16*>(a.Y) + head, head_bytes);
    const auto rV = rsrc(V, head_bytes);
    const auto rP2 = rsrc(P2, head_bytes);
    const int qoff = qrow * (DR * 2) + hf * 16;
    float dyy = 0.0f, dyv = 0.0f, p12 = 0.0f;
#pragma unroll
    for (int ds = 0; ds < DR / 16; ++ds) {
      const bf16x8 y = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rY, qoff + ds * 32, 0, 0));
      const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rV, qoff + ds * 32, 0, 0));
      const bf16x8 p = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP2, qoff + ds * 32, 0, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dyy = fmaf((float)yf[ds][e], (float)y[e], dyy);
        dyv = fmaf((float)yf[ds][e], (float)v[e], dyv);
        p12 = fmaf((float)qf[ds][e], (float)p[e], p12);
      }
    }
    dyy = lane_pair_sum(dyy);
    dyv = lane_pair_sum(dyv);
    p12 = lane_pair_sum(p12);
    float st[4] = {INFINITY, 0.0f, 0.0f, 0.0f};
    if (valid) {
      const float lse = a.lse[(size_t)bh * T + qrow];
      const float logi = logf((float)(qrow + 1));
      const float inv_tau = hp.inv_tau[bh % a.H];
      const float u = p12 * hp.scale;                  // U_ii
      const float S = sigmoid_f32(u * inv_tau);
      const float Fs = expf(S - lse);                  // F_ii
      const float dR = Fs * (dyv - dyy);               // dR_ii
      const float sp = S * (1.0f - S);
      L2 = (lse + hp.lambda * logi) * kLog2e;
      negD = -dyy;
      us = dR * sp * inv_tau * hp.scale;
      st[0] = L2;
      st[1] = negD;
      st[2] = Fs;
      st[3] = us;
      if (hf == 0) {
        ptau = dR * sp * (-u * inv_tau * inv_tau);
        plam = logi * dR;
      }
    }
    if (hf == 0 && qrow < nt * kStatRows) {
#pragma unroll
      for (int k = 0; k < 4; ++k) a.stats[stat_at(bh, nt, qrow, k)] = st[k];
    }
  }
  f32x16 negDv;                                       // G^T accumulators start at -D_q
#pragma unroll
  for (int r = 0; r < 16; ++r) negDv[r] = negD;
  const float c = hp.scale;
  const float k2 = c * kLog2e;

  // Keys 0 .. kend-1 are history for some row of this work-group; tiles
  // before q0 / 64 are strictly left of every row of it.
  const int kend = min(q0 + kDqRows, T) - 1;
  const int ntiles = (kend + kTileRows - 1) / kTileRows;
  const int nsteady = min(ntiles, q0 / kTileRows);

  // Staging: wave w moves blocks w + 8 u of each of the three layouts.
  const int hb = (int)head_bytes;
  int src_row[C::kPer], src_tr[C::kPer];
#pragma unroll
  for (int u = 0; u < C::kPer; ++u) {
    src_row[u] = C::template row_src_real<DR>(wave + kDqWaves * u, lane);
    src_tr[u] = C::template tr_src_real<DR>(wave + kDqWaves * u, lane);
  }
  auto dma = [&](int t) {
    const int left = hb - t * kTileRows * DR * 2;
    const auto rk = rsrc_words(P2 + (size_t)t * kTileRows * DR, left);
    const auto rv = rsrc_words(V + (size_t)t * kTileRows * DR, left);
    char* slot = smem + (t % kDqSlots) * C::kSlotBytes;
#pragma unroll
    for (int u = 0; u < C::kPer; ++u) {
      const int k = wave + kDqWaves * u;
      dma16(rk, slot + k * C::kKBlock, src_row[u]);
      dma16(rv, slot + C::kKBytes + k * C::kKBlock, src_row[u]);
      dma16(rk, slot + 2 * C::kKBytes + k * C::kVBlock, src_tr[u]);
    }
  };
  const int row_base = C::row_base(lane);
  const int tr_even = C::tr_base(lane, false), tr_odd = C::tr_base(lane, true);

  f32x16 acc[C::kDb];
#pragma unroll
  for (int db = 0; db < C::kDb; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // One key tile: publish it, refill the slot read two tiles ago, then
  // evidence, weights and transport per 32-key block. Steady tiles (every
  // block strictly left of every row) skip the block modes and masks.
  auto tile = [&](int t, auto steady) __attribute__((always_inline)) {
    if (t + 1 < ntiles) wait_vm_lgkm<C::kDmaTile, 15>();
    else wait_vm_lgkm<0, 15>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Slot (t + 2) % 3 was last read in iteration t - 1, which every wave has
    // finished once it passed the barrier above.
    if (t + 2 < ntiles) dma(t + 2);
    unsigned so = (unsigned)((t % kDqSlots) * C::kSlotBytes);
    unsigned ok = so + row_base, ov = so + C::kKBytes + row_base;
    unsigned oe = so + 2 * C::kKBytes + tr_even, oo = so + 2 * C::kKBytes + tr_odd;
    asm volatile("" : "+v"(ok), "+v"(ov), "+v"(oe), "+v"(oo));
    const VBase p2t{smem + oe, smem + oo};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bool diag = false;
      if constexpr (!decltype(steady)::value) {
        const int md = mode_keys_below(2 * t + kb, own);
        if (md == 0) continue;
        diag = md == 2;
      }
      const f32x16 s = evidence_block<D>(smem + ok, kb, qf);
      const f32x16 g = evidence_block_from<D>(smem + ov, kb, yf, negDv);
      u32x4 pw[2];
      dq_weights(s, g, k2, c, L2, diag, hf, lq, pw);
      transport_block<D>(p2t, kb, pw, acc);
    }
  };

  if (ntiles > 0) dma(0);
  if (ntiles > 1) dma(1);
  int t = 0;
  for (; t < nsteady; ++t) tile(t, Tag<true>{});
  for (; t < ntiles; ++t) tile(t, Tag<false>{});

  // The chunk's (dtau, dlambda) partial: a fixed-order sum over the rows.
  {
    __shared__ float red[2][kDqWaves];
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) {
      ptau += __shfl_xor(ptau, w, 64);
      plam += __shfl_xor(plam, w, 64);
    }
    if (lane == 0) {
      red[0][wave] = ptau;
      red[1][wave] = plam;
    }
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f, l = 0.0f;
      for (int w = 0; w < kDqWaves; ++w) {
        t += red[0][w];
        l += red[1][w];
      }
      a.part[((size_t)bh * nq + qt) * 2 + 0] = t;
      a.part[((size_t)bh * nq + qt) * 2 + 1] = l;
    }
  }

  if (!valid) return;
  // dP1_i = (sum_j dU_ij p2_j + dU_ii p2_i) / sqrt(d_h); us holds
  // dU_ii / sqrt(d_h). Lane holds columns 32 db + 8 g4 + 4 hf + 0..3.
  const size_t ro = (size_t)qrow * DR;
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      if (32 * db + 8 * g4 >= DR) continue;          // padded columns
      const int col = 32 * db + 8 * g4 + 4 * hf;
      float p[4];
      load4(P2 + ro + col, p);
      const int r = 4 * g4;
      store4(dP1 + ro + col, fmaf(acc[db][r + 0], c, us * p[0]), fmaf(acc[db][r + 1], c, us * p[1]),
             fmaf(acc[db][r + 2], c, us * p[2]), fmaf(acc[db][r + 3], c, us * p[3]));
    }
  }
}

// ---- query gradient from the stored dU --------------------------------------
//
// dP1^T[d][q] += P2^T[d][key] dU^T[key][q] over the blocks the key/value
// kernel stored: the dq kernel's transport (P2 in the transposed layout, one
// barrier per 64-key tile), with its B operand read from the stored blocks
// instead of formed from recomputed evidence. A stored block holds, in lane
// L = 16 lj + k of the wave that formed it, the dU of key k for the queries
// 16 h + 4 lj + 0..3 (h = 0, 1) as two 8-byte halves. A transposing LDS read
// in which lane m of group g addresses key 8 half + 4 (g / 2) + m / 4 at the
// queries 16 (g % 2) + 4 (m % 4) .. +3 gives lane 16 (g % 2) + m the dU of its
// query for four consecutive keys: the operand order of the transport (keys
// 16 ks + 4 (l / 32) + 0..3 and 16 ks + 8 + 4 (l / 32) + 0..3 of a 32-key
// block). Each wave stages its own blocks next to the shared P2 tile.
constexpr int kDuWaveTile = 4 * kDuBlockBytes;     // one wave's blocks of a 64-key tile

template <int D>
struct DquCfg : TileLayout<D> {
  using L = TileLayout<D>;
  static constexpr int kSlotBytes = L::kVBytes + kDqWaves * kDuWaveTile;
  static constexpr int kLdsBytes = kDqSlots * kSlotBytes;
  static constexpr int kPer = L::kBlocks / kDqWaves;   // P2 blocks per wave and tile
  static constexpr int kDmaTile = kPer + 4;            // direct loads per wave and tile
};

template <int D, int DR = D>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dqu_kernel(BwdArgs a, HeadParams hp) {
  static_assert(DR % 16 == 0 && DR <= D && DR >= 32, "real head size within the layout");
  using C = DquCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];

  const int T = a.T;
  const int nq = (T + kDqRows - 1) / kDqRows;
  const int BH = a.B * a.H;
  const int qt = nq - 1 - (int)blockIdx.x / BH;       // longest histories first
  const int bh = (int)blockIdx.x % BH;
  const int nt = (T + kStatRows - 1) / kStatRows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;

  const size_t head = (size_t)bh * (size_t)T * DR;
  const long long head_bytes = (long long)T * DR * 2;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  __bf16* dP1 = static_cast<__bf16*>(a.dP1) + head;

  const int q0 = qt * kDqRows;
  const int qrow = q0 + wave * 32 + lq;               // may be >= T: stores drop
  const int own = q0 / 32 + wave;                     // the wave's 32-query block
  const int kend = min(q0 + kDqRows, T) - 1;
  const int ntiles = (kend + kTileRows - 1) / kTileRows;
  const int nsteady = min(ntiles, q0 / kTileRows);

  const int hb = (int)head_bytes;
  int src_tr[C::kPer];
#pragma unroll
  for (int u = 0; u < C::kPer; ++u) src_tr[u] = C::template tr_src_real<DR>(wave + kDqWaves * u, lane);
  // This wave's stored blocks (own, kb), kb = 0 .. 2 own + 1, lie one after
  // another; blocks past the last one read as zeros (and are never used).
  const int du_bytes = (int)bwd_du_head_bytes(T);
  const u32x4 rdu = rsrc_words(static_cast<const char*>(a.du) + (size_t)bh * (size_t)du_bytes, du_bytes);
  const long long du_src = (long long)own * (own + 1) * kDuBlockBytes + 16 * lane;
  const int kb_last = 2 * own + 1;
  auto dma = [&](int t) {
    const int left = hb - t * kTileRows * DR * 2;
    const auto rk = rsrc_words(P2 + (size_t)t * kTileRows * DR, left);
    char* slot = smem + (t % kDqSlots) * C::kSlotBytes;
#pragma unroll
    for (int u = 0; u < C::kPer; ++u) dma16(rk, slot + (wave + kDqWaves * u) * C::kVBlock, src_tr[u]);
    char* mine = slot + C::kVBytes + wave * kDuWaveTile;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int kb = 4 * t + b;
      const long long o = du_src + (long long)kb * kDuBlockBytes;
      dma16_nt(rdu, mine + b * kDuBlockBytes, kb <= kb_last && o < du_bytes ? (int)o : kOutOfRange);
    }
  };
  const int tr_even = C::tr_base(lane, false), tr_odd = C::tr_base(lane, true);
  const int tg = lane >> 4, tm = lane & 15;
  const int du_lane = (16 * (tm & 3) + 4 * (tg >> 1) + (tm >> 2)) * 16 + 8 * (tg & 1);

  f32x16 acc[C::kDb];
#pragma unroll
  for (int db = 0; db < C::kDb; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  auto tile = [&](int t, auto steady) __attribute__((always_inline)) {
    if (t + 1 < ntiles) wait_vm_lgkm<C::kDmaTile, 15>();
    else wait_vm_lgkm<0, 15>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Slot (t + 2) % 3 was last read in iteration t - 1.
    if (t + 2 < ntiles) dma(t + 2);
    const unsigned so = (unsigned)((t % kDqSlots) * C::kSlotBytes);
    unsigned oe = so + tr_even, oo = so + tr_odd;
    unsigned od = so + C::kVBytes + wave * kDuWaveTile + du_lane;
    asm volatile("" : "+v"(oe), "+v"(oo), "+v"(od));
    const VBase p2t{smem + oe, smem + oo};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!decltype(steady)::value) {
        if (mode_keys_below(2 * t + kb, own) == 0) continue;
      }
      u32x4 pw[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* p = smem + od + (2 * kb + ks) * kDuBlockBytes;
        const bf16x4 lo = lds_tr_read(p), hi = lds_tr_read(p + 128);
        pw[ks] = __builtin_bit_cast(u32x4, bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
      transport_block<D>(p2t, kb, pw, acc);
    }
  };

  if (ntiles > 0) dma(0);
  if (ntiles > 1) dma(1);
  int t = 0;
  for (; t < nsteady; ++t) tile(t, Tag<true>{});
  for (; t < ntiles; ++t) tile(t, Tag<false>{});

  if (qrow >= T) return;
  // dP1_i = (sum_j dU_ij p2_j + dU_ii p2_i) / sqrt(d_h), dU_ii / sqrt(d_h)
  // from the row statistics. Lane holds columns 32 db + 8 g4 + 4 hf + 0..3.
  const float c = hp.scale;
  const float us = a.stats[stat_at(bh, nt, qrow, 3)];
  const size_t ro = (size_t)qrow * DR;
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      if (32 * db + 8 * g4 >= DR) continue;          // padded columns
      const int col = 32 * db + 8 * g4 + 4 * hf;
      float p[4];
      load4(P2 + ro + col, p);
      const int r = 4 * g4;
      store4(dP1 + ro + col, fmaf(acc[db][r + 0], c, us * p[0]), fmaf(acc[db][r + 1], c, us * p[1]),
             fmaf(acc[db][r + 2], c, us * p[2]), fmaf(acc[db][r + 3], c, us * p[3]));
    }
  }
}

// ---- key/value gradients ----------------------------------------------------
//
// v_mfma_f32_16x16x32_bf16 operand layouts (lane l, element e, register r):
//   A (16 x 32): lane l holds A[l % 16][8 (l / 16) + e]
//   B (32 x 16): lane l holds B[8 (l / 16) + e][l % 16]
//   C (16 x 16): lane l, register r holds C[4 (l / 16) + r][l % 16]
// ds_read_b64_tr_b16: when lane m of a 16-lane group addresses row R_{m/4} at
// columns 4 (m % 4) .. +3 of a 16-column span, lane i receives element i of
// the span from rows R_0 .. R_3. Both were established by a probe.
//
// Each wave owns 16 keys and both of their accumulators (dV^T and dP2^T, d_h x
// 16 each), so no operand changes hands between waves. Per 64-query tile and
// 16-query block qb: U[q][key] = P1 . P2^T and G[q][key] = dY . V^T (A read
// row-wise from LDS, the keys' P2 / V rows in registers as B); the C layout
// puts queries 16 qb + 4 (l / 16) + r, key l % 16 in lane l. Two blocks
// (qb0, qb1) then form one transport k-step: with the contraction index
// permuted as {16 qb0 + 4 j + r, 16 qb1 + 4 j + r} for lane group j, the B
// operand F[q][key] (or W) is the lane's own 8 weights, and the A operand
// dY^T[d][q] (or P1^T) is two transposing reads of the same row layout. So a
// tile needs P1 and dY in one layout only, and a ring of 4 tiles (132 KB at
// d_h = 128) needs one barrier per pair of tiles.
// The row layout here packs its 8-row blocks 1024 bytes apart (the forward's
// 1152-byte stride suits the 32x32x16 read pattern only). Measured on gfx950:
// a 16-byte LDS read serves, in each pass, the lane groups {0-7, 24-31},
// {8-15, 16-23} and the same of the upper 32 lanes; with the 1152-byte stride
// the 16x16x32 A-operand read puts both groups of every pass on the same
// banks (two-way conflicts, half the throughput), with 1024 bytes they fall
// in opposite halves. The transposing reads are conflict-free with either.
constexpr int kKvSlots = 4;

template <int D>
struct KvCfg : TileLayout<D> {
  using L = TileLayout<D>;
  static constexpr int kBlk = 1024;                    // block stride of this layout
  static constexpr int kTileBytes = L::kBlocks * kBlk;
  // Waves per work-group (16 keys each): d_h = 128 takes 12 (three per SIMD
  // in one work-group per CU, as the 132 KB ring admits); d_h = 64 takes 8,
  // and its 68 KB ring lets two work-groups share a CU.
  static constexpr int kWaves = D == 128 ? 12 : 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKeys = 16 * kWaves;    // keys per work-group
  // Slot: [P1 row layout][dY row layout][statistics, 1 KB].
  static constexpr int kStatOff = 2 * kTileBytes;
  static constexpr int kSlotBytes = kStatOff + kStatTile * 4;
  static constexpr int kLdsBytes = kKvSlots * kSlotBytes;
  // Wave w moves blocks w, w + kWaves, ... of each tensor's tile (wave 0
  // also the statistics).
  static constexpr int kPer = (L::kBlocks + kWaves - 1) / kWaves;
  static constexpr int kKs = D / 32;           // evidence k-steps
  static constexpr int kDb = D / 16;           // 16-row blocks of the transports
  // Byte offset of (row q, 16-byte chunk c) in a tile (blocks as in the
  // forward's row layout: block q / 8 + 8 (c / 8), position q % 8 + 8 (c % 8)):
  //   kBlk (q / 8 + 8 (c / 8)) + 16 (q % 8 + 8 (c % 8)).
  // Evidence A operand: row 16 qb + l % 16, chunk 4 ks + l / 16.
  __device__ static int e_base(int lane) {
    const int q = lane & 15, c = lane >> 4;
    return kBlk * (q >> 3) + 16 * ((q & 7) + 8 * c);
  }
  static constexpr int e_imm(int qb, int ks) { return 2 * kBlk * qb + 8 * kBlk * (ks / 2) + 512 * (ks % 2); }
  // Transposing read: lane m of group j addresses row 16 qb + 4 j + m / 4,
  // columns 16 db + 4 (m % 4) .. +3 (8 bytes; half m % 2 of chunk 2 db + (m % 4) / 2).
  __device__ static int t_base(int lane) {
    const int m = lane & 15, q = 4 * (lane >> 4) + (m >> 2), c = (m & 3) >> 1;
    return kBlk * (q >> 3) + 16 * ((q & 7) + 8 * c) + 8 * (m & 1);
  }
  static constexpr int t_imm(int qb, int db) { return 2 * kBlk * qb + 8 * kBlk * (db / 4) + 256 * (db % 4); }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 tr_pair(const char* a, const char* b) {
  const bf16x4 x = lds_tr_read(a), y = lds_tr_read(b);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// kDU: also store the packed dU of every processed (32-query, 16-key) pair
// as block (qp, kb) of the stored-dU triangle, for bwd_dqu_kernel.
template <int D, int DR = D, bool kDU = false>
__global__ __launch_bounds__(KvCfg<D>::kThreads, 1) void bwd_dkv_kernel(BwdArgs a, HeadParams hp) {
  static_assert(DR % 16 == 0 && DR <= D && DR >= 32, "real head size within the layout");
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];

  const int T = a.T;
  const int BH = a.B * a.H;
  const int kt = (int)blockIdx.x / BH;                 // earliest keys (longest futures) first
  const int bh = (int)blockIdx.x % BH;
  const int nt = (T + kStatRows - 1) / kStatRows;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int lj = lane >> 4;

  const size_t head = (size_t)bh * (size_t)T * DR;
  const long long head_bytes = (long long)T * DR * 2;
  const __bf16* P1 = static_cast<const __bf16*>(a.P1) + head;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  const __bf16* dY = static_cast<const __bf16*>(a.dY) + head;
  const float* stats = a.stats + (size_t)bh * nt * kStatTile;

  const int k0 = kt * C::kKeys;
  const int kq = k0 + 16 * wave;                       // this wave's 16 keys
  const int kblk = kq / 16;
  const float c = hp.scale;
  const float k2 = c * kLog2e;

  // The keys' P2 and V rows as B operands: lane l holds key kq + l % 16,
  // columns 32 ks + 8 (l / 16) .. +7 (keys >= T and pad columns read 0).
  bf16x8 kf[C::kKs], vf[C::kKs];
  {
    const auto rP2 = rsrc(P2, head_bytes);
    const auto rV = rsrc(V, head_bytes);
#pragma unroll
    for (int ks = 0; ks < C::kKs; ++ks) {
      const int cc = 4 * ks + lj;
      const int o = cc < DR / 8 ? (kq + l16) * (DR * 2) + 16 * cc : kOutOfRange;
      kf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP2, o, 0, 0));
      vf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rV, o, 0, 0));
    }
  }

  // Query tiles t0 .. nt-1 hold every query i > j of this work-group's keys;
  // from ts on, every 16-query block lies strictly below every key block.
  const int t0 = k0 / kTileRows;
  const int ts = (k0 / 16 + C::kWaves - 1) / 4 + 1;
  const int hb = (int)head_bytes;
  int src_row[C::kPer];
#pragma unroll
  for (int u = 0; u < C::kPer; ++u) src_row[u] = C::template row_src_real<DR>(wave + C::kWaves * u, lane);
  auto dma = [&](int t) {
    const int left = hb - t * kTileRows * DR * 2;
    const auto rq = rsrc_words(P1 + (size_t)t * kTileRows * DR, left);
    const auto ry = rsrc_words(dY + (size_t)t * kTileRows * DR, left);
    char* slot = smem + ((t - t0) % kKvSlots) * C::kSlotBytes;
#pragma unroll
    for (int u = 0; u < C::kPer; ++u) {
      const int k = wave + C::kWaves * u;
      if (k < C::kBlocks) {
        dma16(rq, slot + k * C::kBlk, src_row[u]);
        dma16(ry, slot + C::kTileBytes + k * C::kBlk, src_row[u]);
      }
    }
    if (wave == 0) {
      const auto rs = rsrc_words(stats + (size_t)t * kStatTile, kStatTile * 4);
      dma16(rs, slot + C::kStatOff, 16 * lane);
    }
  };
  const int eb = C::e_base(lane);
  const int tb = C::t_base(lane);

  // Stored dU: one 1 KB block per wave and pair of 16-query blocks (lane
  // l's 16 bytes), written as soon as it is formed with the non-temporal
  // hint (it is read once, by the query kernel, and should not push the
  // shared P1 / dY tiles out of the L2).
  const int nqp = (T + 31) / 32;
  const auto rdu = rsrc(kDU ? static_cast<char*>(a.du) + (size_t)bh * (size_t)bwd_du_head_bytes(T) : nullptr,
                        kDU ? bwd_du_head_bytes(T) : 0);

  f32x4 accV[C::kDb], accP[C::kDb];
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
    accV[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    accP[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // The first two query tiles. Tiles go by pairs (t0 + 2n, t0 + 2n + 1):
  // at the start of a pair the waves wait for its loads and meet, then load
  // the next pair into the slots of the previous one; so one barrier serves
  // two tiles. The full wait before the loop covers the key rows too: the
  // compiler sees only the key-row loads (the direct loads are inline
  // assembly), and once it knows they have completed it puts no wait of its
  // own inside the loop, where any vmcnt wait would also stall on the tiles
  // in flight.
  if (t0 < nt) dma(t0);
  if (t0 + 1 < nt) dma(t0 + 1);
  wait_vm_lgkm<0, 15>();

  auto tile = [&](int t, auto steady) __attribute__((always_inline)) {
    if (((t - t0) & 1) == 0) {
      wait_vm_lgkm<0, 15>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 2 < nt) dma(t + 2);
      if (t + 3 < nt) dma(t + 3);
    }
    const unsigned so = (unsigned)(((t - t0) % kKvSlots) * C::kSlotBytes);
    unsigned oe1 = so + eb, oe2 = so + C::kTileBytes + eb;  // P1 / dY evidence reads
    unsigned ot1 = so + tb, ot2 = so + C::kTileBytes + tb;  // P1 / dY transposing reads
    asm volatile("" : "+v"(oe1), "+v"(oe2), "+v"(ot1), "+v"(ot2));
    const float* st = reinterpret_cast<const float*>(smem + so + C::kStatOff);
    int md[4] = {1, 1, 1, 1};                           // 0 none, 1 all, 2 diagonal
    if constexpr (!decltype(steady)::value) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) md[qb] = mode_queries_above(4 * t + qb, kblk);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (md[2 * p] == 0 && md[2 * p + 1] == 0) continue;
      // Evidence of both blocks, then the first transport operands (their
      // LDS latency runs under the weights' VALU work), then the weights,
      // then the transports with each operand read one d-block ahead.
      f32x4 u[2], g[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qb = 2 * p + h;
        u[h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        g[h] = *reinterpret_cast<const f32x4*>(st + kStatRows + 16 * qb + 4 * lj);   // -D_q
        if (md[qb] != 0) {
#pragma unroll
          for (int ks = 0; ks < C::kKs; ++ks) {
            const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(smem + oe1 + C::e_imm(qb, ks));
            const bf16x8 x2 = *reinterpret_cast<const bf16x8*>(smem + oe2 + C::e_imm(qb, ks));
            u[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, kf[ks], u[h], 0, 0, 0);
            g[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x2, vf[ks], g[h], 0, 0, 0);
          }
        }
      }
      bf16x8 ay = tr_pair(smem + ot2 + C::t_imm(2 * p, 0), smem + ot2 + C::t_imm(2 * p + 1, 0));
      bf16x8 ap = tr_pair(smem + ot1 + C::t_imm(2 * p, 0), smem + ot1 + C::t_imm(2 * p + 1, 0));
      u32x4 pf, pw;                                     // packed F and W of blocks 2p, 2p+1
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qb = 2 * p + h;
        float f[4] = {0.0f, 0.0f, 0.0f, 0.0f}, w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (md[qb] != 0) {
          const f32x4 L2 = *reinterpret_cast<const f32x4*>(st + 16 * qb + 4 * lj);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const Terms tm(u[h][r], k2, c, L2[r]);
            float F = tm.F;
            if (md[qb] == 2) F = l16 < 4 * lj + r ? F : 0.0f;   // key < query within the diagonal block
            f[r] = F;
            w[r] = F * g[h][r] * tm.dsilu;
          }
        }
        pf[2 * h + 0] = pack_bf16(f[0], f[1]);
        pf[2 * h + 1] = pack_bf16(f[2], f[3]);
        pw[2 * h + 0] = pack_bf16(w[0], w[1]);
        pw[2 * h + 1] = pack_bf16(w[2], w[3]);
      }
      if constexpr (kDU) {
        const int qp = 2 * t + p;
        if (qp < nqp)
          __builtin_amdgcn_raw_buffer_store_b128(pw, rdu, (qp * (qp + 1) + kblk) * kDuBlockBytes + 16 * lane, 0,
                                                 kCachePolicyNT);
      }
      const bf16x8 bF = __builtin_bit_cast(bf16x8, pf), bW = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < C::kDb; ++db) {
        bf16x8 ny = ay, np = ap;
        if (db + 1 < C::kDb) {
          ny = tr_pair(smem + ot2 + C::t_imm(2 * p, db + 1), smem + ot2 + C::t_imm(2 * p + 1, db + 1));
          np = tr_pair(smem + ot1 + C::t_imm(2 * p, db + 1), smem + ot1 + C::t_imm(2 * p + 1, db + 1));
        }
        accV[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ay, bF, accV[db], 0, 0, 0);
        accP[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bW, accP[db], 0, 0, 0);
        ay = ny;
        ap = np;
      }
    }
  };

  int t = t0;
  for (; t < min(ts, nt); ++t) tile(t, Tag<false>{});
  for (; t < nt; ++t) tile(t, Tag<true>{});

  const int krow = kq + l16;
  if (krow >= T) return;
  const size_t ro = (size_t)krow * DR;
  // accV[db][r] = dV^T[16 db + 4 lj + r][key]: 4 consecutive columns of the key's row.
  // dV_j = sum_i F_ij dY_i + F_jj dY_j;  dP2_j = (sum_i dU_ij p1_i + dU_jj p1_j) / sqrt(d_h).
  __bf16* dV = static_cast<__bf16*>(a.dV) + head;
  __bf16* dP2 = static_cast<__bf16*>(a.dP2) + head;
  const float fs = stats[stat_at(0, nt, krow, 2)];
  const float us = stats[stat_at(0, nt, krow, 3)];
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
    if (16 * db >= DR) continue;                       // padded columns
    const int col = 16 * db + 4 * lj;
    float y[4], q[4];
    load4(dY + ro + col, y);
    load4(P1 + ro + col, q);
    store4(dV + ro + col, fmaf(fs, y[0], accV[db][0]), fmaf(fs, y[1], accV[db][1]), fmaf(fs, y[2], accV[db][2]),
           fmaf(fs, y[3], accV[db][3]));
    store4(dP2 + ro + col, fmaf(accP[db][0], c, us * q[0]), fmaf(accP[db][1], c, us * q[1]),
           fmaf(accP[db][2], c, us * q[2]), fmaf(accP[db][3], c, us * q[3]));
  }
}

template <int D, int DR = D>
hipError_t launch_typed(const BwdArgs& a, const HeadParams& hp, hipStream_t s) {
  const int BH = a.B * a.H;
  const int nq = (a.T + kDqRows - 1) / kDqRows;
  using Ckv = KvCfg<D>;
  const int nk = (a.T + Ckv::kKeys - 1) / Ckv::kKeys;
  if (a.du != nullptr) {
    // Stored dU: the row statistics first, then dkv (which also stores dU),
    // then dP1 as a product over the stored blocks.
    hipError_t e = launch_bwd_prep(a, hp, true, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkv_kernel<D, DR, true>), dim3(nk * BH), dim3(Ckv::kThreads), 0, s, a, hp);
    hipLaunchKernelGGL((bwd_dqu_kernel<D, DR>), dim3(nq * BH), dim3(kDqThreads), 0, s, a, hp);
    return hipGetLastError();
  }
  // dq first: it writes the row statistics that dkv reads.
  hipLaunchKernelGGL((bwd_dq_kernel<D, DR>), dim3(nq * BH), dim3(kDqThreads), 0, s, a, hp);
  hipLaunchKernelGGL((bwd_dkv_kernel<D, DR>), dim3(nk * BH), dim3(Ckv::kThreads), 0, s, a, hp);
  return hipGetLastError();
}

}  // namespace

bool bwd_mfma_supported(int d_h, int T) {
  // Buffer descriptors address one head with 31-bit byte offsets, including
  // the rows past T of the last tile.
  return (d_h == 32 || d_h == 48 || d_h == 64 || d_h == 80 || d_h == 128) && ((long long)T + kDqRows) * d_h * 2 < 0x7fffffffLL;
}

bool bwd_du_supported(int d_h, int T) {
  return bwd_mfma_supported(d_h, T) && bwd_du_head_bytes(T) < 0x7fff0000LL;
}

hipError_t launch_bwd_mfma_bf16(const BwdArgs& a, const HeadParams& hp, hipStream_t s) {
  switch (a.d_h) {
    case 32: return launch_typed<64, 32>(a, hp, s);
    case 48: return launch_typed<64, 48>(a, hp, s);
    case 64: return launch_typed<64>(a, hp, s);
    case 80: return launch_typed<128, 80>(a, hp, s);
    case 128: return launch_typed<128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

// bf16 MFMA FlashRelation forward for gfx950 ("Ask Self, Ask Others: Relation
// Is All You Need", Sec. 5.1, Eq. (12)-(14); App. A.3).
//
// A persistent work-group (8 waves, one per compute unit) takes work items of
// two query tiles of one head, 256 rows each; each wave owns 32 rows and two
// waves share a SIMD. Key tiles of 64 rows of P2 and V are moved by direct
// global->LDS loads into rings of 3 (P2) and 4 (V) slots shared by the 8
// waves; buffer descriptors zero-fill rows >= T.
//
// Per 64-key tile and wave the work is
//   evidence  S^T[key][query] = P2 . P1^T   (v_mfma_f32_32x32x16_bf16; the
//             transposed product puts one query per lane, so a row's scores
//             sit in one lane pair (l, l^32));
//   scan      Exchange weights p = exp(SiLU(u) - m) for keys j < i only (Self is
//             not part of the scan), in the log2 domain:
//             a = u log2 e, SiLU(u) log2 e = a / (1 + 2^-a); weights go to bf16
//             for the transport and the row sum is accumulated in fp32;
//   transport O^T[d][query] += V^T . P^T   (V^T operands come straight from
//             the LDS tile via ds_read_b64_tr_b16).
// The three are software-pipelined across tiles: in iteration j the matrix
// cores run the transport of tile j-1 and the evidence of tile j+1 while the
// VALU forms the stabiliser and then the weights of tile j. In the steady
// state the issue order is fixed in half-steps of 2 MFMAs, each with a slice
// of the VALU work and the LDS reads of the operands two half-steps ahead.
// Steady and boundary (diagonal) iterations run in separate loops; each
// iteration ends with one barrier that publishes the tiles loaded one
// iteration earlier.
//
// Stabiliser: m (log2 domain) starts at 0, which is valid because
// SiLU(u) <= max(u, 0) and SiLU >= -0.2785, so the largest weight of a
// non-empty history is >= e^-0.2785; m moves only when a tile's maximum
// exceeds it by > 8 (lazy rescaling, weights stay <= 2^8).
// Self entry S_i = sigmoid(U_ii / tau) from p1_i . p2_i in fp32 (prologue),
// count term lambda log i, and the branch-free Self/Exchange combination in
// the epilogue, with V_i read from the V ring; the first row gets Y_1 = V_1
// exactly.
//
// Causal tile skip: a work-group scans only key tiles left of its last row;
// near the diagonal a wave skips 32-key blocks right of its diagonal block and
// masks keys j >= i inside it.
#include <atomic>
#include <type_traits>

#include "mfma_tile.h"
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

using namespace mfma;

constexpr int kBM = 256;          // query rows per work-group
constexpr int kBN = kTileRows;    // keys per LDS tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKSlots = 3;        // LDS ring depth of P2 (tile t in slot t % 3)
constexpr int kVSlots = 4;        // LDS ring depth of V (tile t in slot t % 4)
constexpr float kLazy = 8.0f;     // rescale only when the max grows by > 2^8

// Block modes of a 64-key tile for one wave (blocks kb0 = keys 0..31, kb1 = 32..63).
enum : int {
  kFull = 0,   // both blocks strictly left of the wave's rows
  kDiag1 = 1,  // kb0 full, kb1 is the wave's diagonal block
  kDiag0 = 2,  // kb0 is the diagonal block, kb1 lies to the right
  kOff = 3     // the whole tile lies to the right (or past the history)
};

// P2 tiles are kept in the row layout (evidence operands), V tiles in the
// transposed layout (transport operands).
template <int D>
struct Cfg : TileLayout<D> {
  using L = TileLayout<D>;
  // + one block that absorbs direct loads of V tiles past the last one needed.
  static constexpr int kLdsBytes = kKSlots * L::kKBytes + kVSlots * L::kVBytes + L::kVBlock;
  static constexpr int kDmaPerWave = L::kBlocks / kWaves;   // blocks per wave per tile and operand
  static constexpr int kPV = 2 * 2 * L::kDb;                // transport MFMAs per tile
  static constexpr int kQK = 2 * L::kDs;                    // evidence MFMAs per tile
  static constexpr int kSteps = (kPV + kQK) / 4;            // steady-state steps
  static_assert(kPV >= 4 && (kPV + kQK) % 4 == 0, "step layout");
  static_assert(kPV == 4 * (kSteps / 2) && kSteps >= 4, "evidence chains start at step kSteps / 2");
  static_assert(L::kBlocks % kWaves == 0, "each wave moves whole blocks");
};

// Work item w = (b*H + h, pair pr): the query tiles nq-1-pr and pr of one
// head, which together scan the same number of key tiles, so every item costs
// the same. Work-groups are dealt to the 8 XCDs round-robin and a work-group
// takes items w = blockIdx.x + k * gridDim.x; when both gridDim.x and B*H are
// multiples of 8, the items an XCD runs all come from its own eighth of the
// heads, so their P2/V stay in that XCD's L2.
__device__ __forceinline__ void work_of(int w, int G, int npair, int BH, int& bh, int& pr) {
  if ((BH & 7) == 0 && (G & 7) == 0) {
    const int xcd = w & 7, i = w >> 3;
    bh = xcd * (BH >> 3) + i / npair;
    pr = i % npair;
  } else {
    bh = w / npair;
    pr = w % npair;
  }
}

// Mode of tile t (key blocks 2t, 2t+1) for the wave whose diagonal block is dblk.
__device__ __forceinline__ int tile_mode(int t, int ntiles, int dblk) {
  if (t < 0 || t >= ntiles) return kOff;
  const int b0 = 2 * t;
  if (b0 + 1 < dblk) return kFull;
  if (b0 + 1 == dblk) return kDiag1;
  return b0 == dblk ? kDiag0 : kOff;
}

__device__ __forceinline__ bool blk_active(int mode, int kb) {
  return mode == kFull || mode == kDiag1 || (mode == kDiag0 && kb == 0);
}
__device__ __forceinline__ bool blk_diag(int mode, int kb) {
  return (mode == kDiag1 && kb == 1) || (mode == kDiag0 && kb == 0);
}

// Exchange weight of one score (log2 domain): 2^(a / (1 + 2^-a) - m2), a = s k2.
__device__ __forceinline__ float exch_weight(float s, float k2, float m2) {
  const float av = s * k2;
  const float den = 1.0f + __builtin_amdgcn_exp2f(-av);
  return __builtin_amdgcn_exp2f(av * __builtin_amdgcn_rcpf(den) - m2);
}

// Exchange weights of one 32-key block into packed bf16 transport operands
// (register r of the evidence tile -> operand r / 8, element r % 8) and the
// row-sum share (fp32 adds into four partial sums).
template <bool kMasked>
__device__ __forceinline__ void weights_block(const f32x16& s, float k2, float m2, int hf, int lq,
                                              u32x4 (&pf)[2], float& lsum) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    float w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      w[e] = exch_weight(s[r + e], k2, m2);
      // Key of register r within the block: 8 (r / 4) + 4 hf + r % 4.
      if (kMasked) w[e] = (8 * ((r + e) >> 2) + 4 * hf + ((r + e) & 3)) < lq ? w[e] : 0.0f;
      acc[(r + e) & 3] += w[e];
    }
    pf[r >> 3][(r & 7) >> 1] = pack_bf16(w[0], w[1]);
  }
  lsum += (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <bool kMasked>
__device__ __forceinline__ float block_max(const f32x16& s, int hf, int lq) {
  // Four independent partial maxima keep the dependency chain short.
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = s[r];
    if (kMasked) x = (8 * (r >> 2) + 4 * hf + (r & 3)) < lq ? x : -INFINITY;
    mx[r & 3] = fmaxf(mx[r & 3], x);
  }
  return fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
}

// Raw Self evidence p1_i . p2_i of the lane's query from its diagonal block's
// evidence tile: register r holds key 8 (r / 4) + 4 hf + r % 4, which is the
// query lq in the half hf = (lq / 4) % 2, register 4 (lq / 8) + lq % 4; the
// other half contributes 0 (the halves are summed at the end).
__device__ __forceinline__ float diag_entry(const f32x16& s, int hf, int lq) {
  const int rs = 4 * (lq >> 3) + (lq & 3);
  float v = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) v = r == rs ? s[r] : v;
  return ((lq >> 2) & 1) == hf ? v : 0.0f;
}

// Lazy stabiliser update from a tile's raw maximum: returns the factor the
// accumulated O and row sum must be multiplied by (1 if m does not move).
__device__ __forceinline__ float stabilise(float mx, float k2, float& m2) {
  mx = lane_pair_max(mx);
  const float mc2 = fmaxf(mx, 0.0f) * k2;
  const float mnew = mc2 > m2 + kLazy ? mc2 : m2;
  const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
  m2 = mnew;
  return alpha;
}

template <int D>
__device__ __forceinline__ void rescale(f32x16 (&o)[D / 32], float alpha) {
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
}

// D: head size of the LDS tile layout and the MFMA schedule (64 or 128); DR:
// the rows' real head size in memory (48 runs on the 64 layout and 80 on the
// 128 layout, the chunks past DR held at zero, so evidence and transport are
// exact and the padded output rows are not stored).
template <int D, int DR = D>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_kernel(FwdArgs a, HeadParams hp) {
  static_assert(DR % 16 == 0 && DR <= D && DR > D / 2, "real head size within the layout");
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];
  char* const kbase = smem;                          // P2 ring: tile t in slot t % 3
  char* const vbase = smem + kKSlots * C::kKBytes;   // V ring:  tile t in slot t % 4

  const int T = a.T;
  const int nq = (T + kBM - 1) / kBM;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;                      // query (column) within the wave
  const int hf = lane >> 5;                      // lane half

  // P1 rows of a query tile as the evidence MFMA's B operand: lane holds
  // p1[qrow][16 ds + 8 hf + 0..7]. They are loaded one tile ahead, before the
  // previous tile's epilogue, so their latency hides behind it.
  bf16x8 qf[C::kDs];
  auto load_q = [&](int qt, int bh) __attribute__((always_inline)) {
    const auto rP1 = rsrc(static_cast<const __bf16*>(a.P1) + (size_t)bh * (size_t)T * DR, (long long)T * DR * 2);
    const int qoff = (qt * kBM + wave * 32 + lq) * (DR * 2) + hf * 16;
#pragma unroll
    for (int ds = 0; ds < C::kDs; ++ds) {
      // k-steps past DR / 16 cover padded columns: out-of-range offsets read 0.
      const int o = ds < DR / 16 ? qoff + ds * 32 : kOutOfRange;
      qf[ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP1, o, 0, 0));
    }
  };

  // One query tile (256 rows) of one head, start to finish; then, when nqt >=
  // 0, the P1 rows of query tile nqt of head nbh are loaded before the
  // epilogue.
  auto run_tile = [&](int qt, int bh, int nqt, int nbh) __attribute__((always_inline)) {
  const int h = bh % a.H;
  const size_t head = (size_t)bh * (size_t)T * DR;
  const long long head_bytes = (long long)T * DR * 2;
  const __bf16* P1 = static_cast<const __bf16*>(a.P1) + head;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  __bf16* Y = static_cast<__bf16*>(a.Y) + head;
  const auto rY = rsrc(Y, head_bytes);

  const int q0 = qt * kBM;
  const int qrow = q0 + wave * 32 + lq;          // may be >= T: loads give 0, stores drop
  const int dblk = q0 / 32 + wave;               // the wave's diagonal 32-key block

  const float inv_tau = hp.inv_tau[h];

  const float k2 = hp.scale * kLog2e;            // raw dot -> log2-domain evidence

  // Keys 0 .. kend-1 are history for some row of this tile.
  const int kend = min(q0 + kBM, T) - 1;
  const int ntiles = (kend + kBN - 1) / kBN;
  // V tiles loaded: every key <= kend, so that the last four (which stay in
  // the ring) hold the V rows of this tile's own queries for the Self term.
  const int nvt = kend / kBN + 1;

  // Staging: wave w moves blocks k = w + 8 u of a P2 tile (row layout) and
  // of a V tile (transposed layout).
  // Tiles past the last one a work-group needs get an empty descriptor: the
  // loads still issue (and write zeros) but move no data from memory.
  const int hb = (int)head_bytes;
  int dma_koff[C::kDmaPerWave], dma_voff[C::kDmaPerWave];
#pragma unroll
  for (int u = 0; u < C::kDmaPerWave; ++u) {
    const int k = wave + kWaves * u;
    dma_koff[u] = C::template row_src_real<DR>(k, lane);
    dma_voff[u] = C::template tr_src_real<DR>(k, lane);
  }
  auto dma_k = [&](int t) {
    const auto rs = rsrc_words(P2 + (size_t)t * kBN * DR, t < ntiles ? hb - t * kBN * DR * 2 : 0);
    char* slot = kbase + (t % kKSlots) * C::kKBytes;
#pragma unroll
    for (int u = 0; u < C::kDmaPerWave; ++u) dma16(rs, slot + (wave + kWaves * u) * C::kKBlock, dma_koff[u]);
  };
  // V tiles past nvt go to the sink block, so the ring keeps the last real ones.
  char* const vsink = vbase + kVSlots * C::kVBytes;
  auto dma_v = [&](int t) {
    const auto rs = rsrc_words(V + (size_t)t * kBN * DR, t < nvt ? hb - t * kBN * DR * 2 : 0);
    char* slot = vbase + (t & (kVSlots - 1)) * C::kVBytes;
#pragma unroll
    for (int u = 0; u < C::kDmaPerWave; ++u)
      dma16(rs, t < nvt ? slot + (wave + kWaves * u) * C::kVBlock : vsink, dma_voff[u]);
  };
  constexpr int kDmaIter = 2 * C::kDmaPerWave;   // direct loads a wave issues per iteration

  // Lane read bases: evidence operand rows of P2 and the transposed V reads.
  const int koff = C::row_base(lane);
  const int voff_even = C::tr_base(lane, false);
  const int voff_odd = C::tr_base(lane, true);
  // Per-lane read bases of the slot holding tile t. The base is formed once
  // per use site in a register (opaque to the optimiser), so every operand
  // read is that register plus an immediate; otherwise the compiler hoists a
  // separate loop-invariant address per immediate and runs out of registers.
  auto kslot = [&](int t) -> const char* {
    unsigned off = (unsigned)(kbase - smem) + (unsigned)((t % kKSlots) * C::kKBytes + koff);
    asm volatile("" : "+v"(off));
    return smem + off;
  };
  auto vslot = [&](int t) -> VBase {
    const unsigned slot = (unsigned)(vbase - smem) + (unsigned)((t & (kVSlots - 1)) * C::kVBytes);
    unsigned e = slot + voff_even, o = slot + voff_odd;
    asm volatile("" : "+v"(e), "+v"(o));
    return VBase{smem + e, smem + o};
  };

  // Prologue: P2 tiles 0..2 and V tiles 0..1 into their slots, evidence of tile 0.
  dma_k(0);
  dma_k(1);
  dma_k(2);
  dma_v(0);
  dma_v(1);
  // Self evidence p1_i . p2_i: the diagonal block's evidence tile provides it
  // (diag_entry) whenever the scan reaches that block. It does not only for a
  // wave whose first row is T - 1 with T - 1 a multiple of 64 (its own key
  // tile holds no history), or whose rows all lie past T; such a wave takes
  // the dot product of the rows.
  float dself = 0.0f;
  if (dblk >= 2 * ntiles) {
    const auto rP2 = rsrc(P2, head_bytes);
    const int qoff = qrow * (DR * 2) + hf * 16;
#pragma unroll
    for (int ds = 0; ds < C::kDs; ++ds) {
      const int o = ds < DR / 16 ? qoff + ds * 32 : kOutOfRange;
      const bf16x8 kv = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP2, o, 0, 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) dself = fmaf((float)qf[ds][e], (float)kv[e], dself);
    }
  }
  wait_vm_lgkm<0, 15>();
  __syncthreads();
  // Evidence of tile j (s_cur, per 32-key block) and packed bf16 weights of
  // tile j-1 (p_prev, per block and MFMA k-step) on entry to iteration j.
  f32x16 s_cur[2];
  u32x4 p_prev[2][2];
  {
    const int md = tile_mode(0, ntiles, dblk);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (blk_active(md, kb)) {
        s_cur[kb] = evidence_block<D>(kslot(0), kb, qf);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s_cur[kb][r] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) p_prev[kb][ks] = u32x4{0u, 0u, 0u, 0u};
  f32x16 o[C::kDb];
#pragma unroll
  for (int db = 0; db < C::kDb; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m2 = 0.0f;                               // stabiliser, log2 domain
  float lsum = 0.0f;                             // this lane's share of the row sum
  constexpr int kRing = 6;                       // operand ring of the steady state:
  bf16x8 fr[kRing];                              // MFMA i reads fr[i % 6]
  // P2 slot 0 is rewritten in iteration 0.
  __syncthreads();

  // Iteration j = 0 .. ntiles (the last one only transports tile ntiles-1).
  // On entry: m2 = m_{j-1}; O holds tiles <= j-2 (at m_{j-1} once rescaled by
  // alpha_prev at the start); the row sum holds tiles <= j-1 at m_{j-1};
  // P2 tile j+1 and V tiles j-1, j are readable in LDS, P2 tile j+2 and V
  // tile j+1 may still be arriving; fr[0..3] hold the first transport
  // operands of the steady state.
  // Every iteration issues the same direct loads and ends with one barrier,
  // whichever of the two bodies a wave runs, so the waves stay matched.
  f32x16 s_next[2];
  u32x4 p_cur[2][2];
  // O is multiplied by alpha_prev = 2^(m_{j-2} - m_{j-1}) at the start of
  // iteration j (before the transport of tile j-1, so that no branch splits
  // the iteration body).
  float alpha_prev = 1.0f;
  // Staging: iteration j issues the direct loads of P2 tile j+3 into the slot
  // of tile j and of V tile j+2 into the slot of tile j-2 (both last read in
  // iteration j-1); the end of iteration j+1 waits for them.
  // Iteration end: read the first transport operands of the next iteration,
  // wait for the previous iteration's direct loads, meet the other waves, and
  // hand the tiles' values on.
  auto finish = [&](int j, float alpha) __attribute__((always_inline)) {
    alpha_prev = alpha;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    {
      const VBase vn = vslot(j);   // V tile j, published by the previous barrier
#pragma unroll
      for (int m = 0; m < 4; ++m) fr[m] = v_operand<D>(vn, m);
    }
    __builtin_amdgcn_sched_barrier(0);
    // All but this iteration's direct loads have landed in LDS once vmcnt is
    // down to kDmaIter (vector memory operations complete in order); the
    // operand reads above (8 LDS reads) may still be in flight.
    wait_vm_lgkm<kDmaIter, 8>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s_cur[kb] = s_next[kb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) p_prev[kb][ks] = p_cur[kb][ks];
    }
  };

  // Boundary / diagonal iteration: per-block activity and masks.
  auto generic_iteration = [&](int j) __attribute__((always_inline)) {
    const char* kl = kslot(j + 1);
    const VBase vl = vslot(j - 1);
    dma_k(j + 3);
    dma_v(j + 2);
    rescale<D>(o, alpha_prev);
    const int md_prev = tile_mode(j - 1, ntiles, dblk);
    const int md_cur = tile_mode(j, ntiles, dblk);
    const int md_next = tile_mode(j + 1, ntiles, dblk);
    float alpha;
    // Phases run in the order that frees registers soonest: the transport
    // releases the previous weights, the weights release this tile's scores
    // before the next tile's evidence is formed.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (blk_active(md_cur, kb))
        mx = fmaxf(mx, blk_diag(md_cur, kb) ? block_max<true>(s_cur[kb], hf, lq) : block_max<false>(s_cur[kb], hf, lq));
    alpha = stabilise(mx, k2, m2);
    lsum *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (blk_active(md_prev, kb)) transport_block<D>(vl, kb, p_prev[kb], o);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (blk_active(md_cur, kb)) {
        if (blk_diag(md_cur, kb)) {
          dself = diag_entry(s_cur[kb], hf, lq);
          weights_block<true>(s_cur[kb], k2, m2, hf, lq, p_cur[kb], lsum);
        } else {
          weights_block<false>(s_cur[kb], k2, m2, hf, lq, p_cur[kb], lsum);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) p_cur[kb][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (blk_active(md_next, kb)) {
        s_next[kb] = evidence_block<D>(kl, kb, qf);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s_next[kb][r] = 0.0f;
      }
    }
    finish(j, alpha);
  };

  // Steady-state iteration (tiles j-1, j, j+1 all strictly left of the wave's
  // rows): half-steps of 2 MFMAs (transport of tile j-1, then evidence of tile
  // j+1), each with a slice of VALU work and the LDS reads of the operands two
  // half-steps ahead. Half-steps 0-1 form tile j's stabiliser; the weights of
  // tile j run as a three-stage pipeline over all half-steps.
  auto steady_iteration = [&](int j) __attribute__((always_inline)) {
    const char* kl = kslot(j + 1);
    const VBase vl = vslot(j - 1);
    dma_k(j + 3);
    dma_v(j + 2);
    rescale<D>(o, alpha_prev);
    float alpha, mx;
    constexpr int kNH = 2 * C::kSteps;           // half-steps
    constexpr int kH = C::kPV / 2;               // first evidence half-step
    auto frag = [&](int i) -> bf16x8 {
      if (i < C::kPV) return v_operand<D>(vl, i);
      const int q = i - C::kPV;
      return *reinterpret_cast<const bf16x8*>(kl + C::k_imm(q / C::kDs, q % C::kDs));
    };
    // Half-steps 0 .. kNS-1 start score pairs; pair n starts in the half-step h
    // with s1_begin(h) <= n < s1_begin(h + 1). Block 0's pairs all start before
    // the evidence chain of the next tile's block 0 (half-step kH), which can
    // then take over their registers.
    constexpr int kNS = kNH - 2;
    auto s1_begin = [](int h) { return 16 * h / kNS; };
    static_assert(16 * kH / kNS >= 8, "block 0 consumed before its registers are reused");
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float av[16][2], rc[16][2];
#pragma unroll
    for (int h = 0; h < kNH; ++h) {
      if (h + 2 < kNH) {
#pragma unroll
        for (int m = 0; m < 2; ++m) fr[(2 * (h + 2) + m) % kRing] = frag(2 * (h + 2) + m);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int i = 2 * h + m;
        const bf16x8 a_op = fr[i % kRing];
        if (i < C::kPV) {
          const int kb = i / (2 * C::kDb), ks = (i / C::kDb) % 2, db = i % C::kDb;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, __builtin_bit_cast(bf16x8, p_prev[kb][ks]), o[db], 0, 0, 0);
        } else {
          const int q = i - C::kPV, kb = q / C::kDs, ds = q % C::kDs;
          if (ds == 0) {
            const f32x16 zero = {};
            s_next[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, qf[0], zero, 0, 0, 0);
          } else {
            s_next[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, qf[ds], s_next[kb], 0, 0, 0);
          }
        }
      }
      if (h == 0) mx = fmaxf(block_max<false>(s_cur[0], hf, lq), block_max<false>(s_cur[1], hf, lq));
      if (h == 1) {
        alpha = stabilise(mx, k2, m2);
        lsum *= alpha;
      }
      // Weights of score pair n (registers 2n, 2n+1 of block n / 8) in three
      // stages over consecutive half-steps, so that the instructions of one
      // half-step do not depend on each other: a = s k2 and 2^-a; then
      // 1 / (1 + 2^-a); then 2^(a / (1 + 2^-a) - m2) (after the stabiliser
      // of half-step 1), its row-sum share and bf16 packing.
      if (h >= 2) {
#pragma unroll
        for (int n = s1_begin(h - 2); n < s1_begin(h - 1); ++n) {
          const int kb = n >> 3, r = 2 * (n & 7);
          const float w0 = __builtin_amdgcn_exp2f(av[n][0] * rc[n][0] - m2);
          const float w1 = __builtin_amdgcn_exp2f(av[n][1] * rc[n][1] - m2);
          acc[r & 3] += w0;
          acc[(r + 1) & 3] += w1;
          p_cur[kb][r >> 3][(r & 7) >> 1] = pack_bf16(w0, w1);
        }
      }
      if (h >= 1 && h - 1 < kNS) {
#pragma unroll
        for (int n = s1_begin(h - 1); n < s1_begin(h); ++n)
#pragma unroll
          for (int e = 0; e < 2; ++e) rc[n][e] = __builtin_amdgcn_rcpf(1.0f + rc[n][e]);
      }
      if (h < kNS) {
#pragma unroll
        for (int n = s1_begin(h); n < s1_begin(h + 1); ++n) {
          const int kb = n >> 3, r = 2 * (n & 7);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            av[n][e] = s_cur[kb][r + e] * k2;
            rc[n][e] = __builtin_amdgcn_exp2f(-av[n][e]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum += (acc[0] + acc[1]) + (acc[2] + acc[3]);
    finish(j, alpha);
  };

  // A wave's steady iterations are j = 1 .. jE-1: tile j+1 must lie strictly
  // left of its diagonal block (2 (j+1) + 1 < dblk) and inside the history.
  const int jE = dblk >= 2 ? max(1, min(ntiles - 1, (dblk - 2) / 2)) : 1;
  generic_iteration(0);
  int j = 1;
  for (; j < jE; ++j) steady_iteration(j);
  for (; j <= ntiles; ++j) generic_iteration(j);
  // The last iterations' direct loads (of tiles past the end) must land
  // before the work-group's LDS is released.
  wait_vm_lgkm<0, 15>();
  if (nqt >= 0) load_q(nqt, nbh);
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue -------------------------------------------------------------
  lsum = lane_pair_sum(lsum);
  dself = lane_pair_sum(dself);
  const float S = sigmoid_f32(dself * hp.scale * inv_tau);
  const RowCombine c(S, m2 * kLn2, lsum, hp.lambda * logf((float)(qrow + 1)));
  if (a.lse != nullptr && hf == 0 && qrow < T) a.lse[(size_t)bh * T + qrow] = c.lse;
  const int roff = qrow * (DR * 2) + hf * 8;
  // V_i of this lane's row from the V ring (tile qrow / 64 is among the last
  // four loaded): columns 32 db + 8 g4 + 4 hf .. +3, i.e. half hf of chunk
  // 4 db + g4 of row qrow % 64 in the block layout.
  bf16x4 vv[C::kDb][4];
  {
    const int r = qrow & (kBN - 1);
    const char* vrow = vbase + ((qrow / kBN) & (kVSlots - 1)) * C::kVBytes + C::kVBlock * (r >> 3) + 8 * hf;
    const int sw = 4 * (((r & 7) >> 1) & 1);
#pragma unroll
    for (int db = 0; db < C::kDb; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = 4 * db + g4;
        vv[db][g4] = *reinterpret_cast<const bf16x4*>(vrow + C::kVBlock * 8 * (c >> 3) + 16 * (8 * (r & 7) + ((c & 7) ^ sw)));
      }
  }
  // Every wave's reads are done before the next tile's loads refill the ring.
  wait_vm_lgkm<63, 0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      if (32 * db + 8 * g4 >= DR) continue;      // padded columns
      bf16x4 yy;
#pragma unroll
      for (int e = 0; e < 4; ++e) yy[e] = (__bf16)(c.w_self * (float)vv[db][g4][e] + c.w_hist * o[db][4 * g4 + e]);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, yy), rY, roff + (32 * db + 8 * g4) * 2, 0, 0);
    }
  }
  };

  const int npair = (nq + 1) / 2;
  const int nwork = a.B * a.H * npair;
  // Item w runs the heavier tile nq-1-pr, then pr (an odd tile count leaves
  // the middle tile alone); each tile names the next one of the work-group.
  int w = blockIdx.x;
  if (w >= nwork) return;
  int bh, pr;
  work_of(w, gridDim.x, npair, a.B * a.H, bh, pr);
  int qt = nq - 1 - pr;
  load_q(qt, bh);
#pragma nounroll
  while (true) {
    int nqt = -1, nbh = bh, npr = pr, nw = w;
    if (qt != pr) {
      nqt = pr;
    } else if (w + (int)gridDim.x < nwork) {
      nw = w + gridDim.x;
      work_of(nw, gridDim.x, npair, a.B * a.H, nbh, npr);
      nqt = nq - 1 - npr;
    }
    run_tile(qt, bh, nqt, nbh);
    if (nqt < 0) break;
    w = nw;
    bh = nbh;
    pr = npr;
    qt = nqt;
  }
}

template <int D, int DR = D>
hipError_t launch_typed(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  const int nq = (a.T + kBM - 1) / kBM;
  const long long nwork = (long long)((nq + 1) / 2) * a.B * a.H;
  if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
  // One persistent work-group per compute unit (the LDS rings admit one).
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const long long grid = nwork < n_cu ? nwork : n_cu;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, DR>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, hp);
  return hipGetLastError();
}

}  // namespace

hipError_t device_cu_count(int* n_cu) {
  // Cached per device; concurrent first calls store the same value.
  static std::atomic<int> cus[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    n = n > 0 ? n : 1;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  *n_cu = n;
  return hipSuccess;
}

bool fwd_mfma_supported(int d_h, int T) {
  // Buffer descriptors address one head with 31-bit byte offsets, including
  // the rows past T of the last query tile.
  return (d_h == 48 || d_h == 64 || d_h == 80 || d_h == 128) && ((long long)T + kBM) * d_h * 2 < 0x7fffffffLL;
}

hipError_t launch_fwd_mfma_bf16(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  switch (a.d_h) {
    case 48: return launch_typed<64, 48>(a, hp, s);
    case 64: return launch_typed<64>(a, hp, s);
    case 80: return launch_typed<128, 80>(a, hp, s);
    case 128: return launch_typed<128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

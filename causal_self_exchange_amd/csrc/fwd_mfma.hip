// bf16 MFMA FlashRelation forward for gfx950 ("Ask Self, Ask Others: Relation
// Is All You Need", Sec. 5.1, Eq. (12)-(14); App. A.3).
//
// A persistent work-group (8 waves, one per compute unit) takes work items of
// two query tiles of one head, 256 rows each; each wave owns 32 query rows and
// two waves share a SIMD. Key tiles of 64 rows of P2 and V are moved by direct
// global->LDS loads into 4-slot rings shared by the 8 waves; buffer
// descriptors zero-fill rows >= T.
//
// Per 32-key block b and wave:
//   evidence  E(b): S^T[key][query] = P2 . P1^T on v_mfma_f32_32x32x16_bf16
//             (the transposed product puts one query per lane, so each lane
//             holds 16 scores of its row);
//   weights   W(b): Exchange weight w = 2^(a sigma(a) - m2) for keys j < i
//             (Self is not part of the scan), a = u log2 e, sigma(a) =
//             1 / (1 + 2^-a): two exponentials and one reciprocal per score,
//             rounded to bf16 pairs for the transport;
//   transport T(b): O^T[d][query] += V^T . W^T (V^T operands straight from
//             the LDS tile via ds_read_b64_tr_b16).
// They run as a software pipeline over blocks: one block step issues the
// MFMAs of E(b+1) and T(b-1), alternating, while the VALU forms W(b) in two
// stages (2^-a and the reciprocal of one score, then the weight of the
// previous one); operand reads run two MFMAs ahead, also across the tile
// barrier. Two block steps make one iteration over a 64-key tile; every
// iteration ends with one barrier.
//
// Two variants share the code:
//   relation_fwd / relation_fwd_ex (kLse = false): P1 is scaled by
//     log2 e / sqrt(d_h) while it is loaded (one bf16 rounding), so the
//     evidence MFMA yields a directly; the row sum is accumulated by a
//     16x16x32 MFMA from the bf16 weights the transport uses, so each row of
//     Y is normalised by exactly the weights it was built from.
//   relation_fwd_lse (kLse = true): a = (p1 . p2) log2 e / sqrt(d_h) in fp32
//     and the row sum from the fp32 weights, so the stored log normaliser
//     keeps full fp32 accuracy for the backward.
//
// Stabiliser: the scan runs with a fixed per-row offset m2 = 0 (log2 domain).
// This is exact whenever nothing overflows: SiLU(u) >= -0.2785, so no weight
// falls below 2^-0.402, and fp32 / bf16 share the 8-bit exponent, so weights
// up to 2^100 and their sums are represented with full relative precision.
// After the scan each wave checks that its row sums stay below 2^100 and that
// O is finite; if any wave of the work-group fails (|U| beyond ~70), the
// work-group redoes the tile: an evidence-only pass finds each row's maximum
// a, then the scan runs again with m2 = max(0, that maximum), so no weight
// exceeds 1.
//
// Self entry S_i = sigmoid(U_ii / tau) with U_ii read out of the diagonal
// block's evidence, the count term lambda log i, and the branch-free
// Self/Exchange combination in the epilogue (Y_1 = V_1 exactly); V_i comes
// from the V ring, whose last four tiles hold the work-group's own rows.
//
// Causal skip: each wave scans key blocks up to its diagonal block (keys
// j >= i masked there) and skips the blocks right of it.
#include <atomic>

#include "mfma_tile.h"
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

using namespace mfma;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;          // query rows per work-group tile
constexpr int kBN = kTileRows;    // keys per LDS tile (two 32-key blocks)
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kKSlots = 4;        // LDS ring depth of P2 (tile t in slot t % 4)
constexpr int kVSlots = 4;        // LDS ring depth of V (tile t in slot t % 4)
constexpr float kFinite = 0x1p100f;   // largest row sum the fixed offset accepts

// P2 tiles are kept in the row layout (evidence operands), V tiles in the
// transposed layout (transport operands).
template <int D>
struct Cfg : TileLayout<D> {
  using L = TileLayout<D>;
  static constexpr int kKRing = kKSlots * L::kKBytes;
  static constexpr int kVRing = kVSlots * L::kVBytes;
  // + one block that absorbs direct loads of V tiles past the last one
  // needed (so the ring keeps the work-group's own rows), + 8 wave flags.
  static constexpr int kLdsBytes = kKRing + kVRing + L::kVBlock + 64;
  static constexpr int kDmaPerWave = L::kBlocks / kWaves;   // blocks per wave per tile and operand
  static constexpr int kSteps = 2 * L::kDs;                 // MFMA steps per block (evidence + transport)
  static constexpr int kScores = 16 / kSteps;               // weights formed per step
  static_assert(L::kBlocks % kWaves == 0, "each wave moves whole blocks");
  static_assert(kSteps % 4 == 0 && 16 % kSteps == 0, "step layout");
  static_assert(2 * L::kDb == L::kDs, "one transport MFMA per evidence MFMA");
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

// Key of register r of an evidence tile within its 32-key block.
__device__ __forceinline__ constexpr int key_of(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

template <bool kMasked>
__device__ __forceinline__ float block_max(const f32x16& s, int hf, int lq) {
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = s[r];
    if (kMasked) x = key_of(r, hf) < lq ? x : -INFINITY;
    mx[r & 3] = fmaxf(mx[r & 3], x);
  }
  return fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
}

// Raw Self evidence of the lane's query from its diagonal block's evidence
// tile: register r holds key 8 (r / 4) + 4 hf + r % 4, which is the query lq
// in the half hf = (lq / 4) % 2, register 4 (lq / 8) + lq % 4; the other
// half contributes 0 (the halves are summed at the end).
__device__ __forceinline__ float diag_entry(const f32x16& s, int hf, int lq) {
  const int rs = 4 * (lq >> 3) + (lq & 3);
  float v = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) v = r == rs ? s[r] : v;
  return ((lq >> 2) & 1) == hf ? v : 0.0f;
}

// Block roles of one step: weights off, full, or on the diagonal block.
enum : int { kWOff = 0, kWFull = 1, kWDiag = 2 };
template <bool kE, int kW, bool kT>
struct StepKind {
  static constexpr bool E = kE;
  static constexpr int W = kW;
  static constexpr bool T = kT;
};

// D: head size of the LDS tile layout and the MFMA schedule (64 or 128); DR:
// the rows' real head size in memory (48 runs on the 64 layout and 80 on the
// 128 layout, the chunks past DR held at zero, so evidence and transport are
// exact and the padded output rows are not stored).
template <int D, int DR, bool kLse>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_kernel(FwdArgs a, HeadParams hp) {
  static_assert(DR % 16 == 0 && DR <= D && DR > D / 2, "real head size within the layout");
  using C = Cfg<D>;
  constexpr int kNS = C::kSteps;
  constexpr int kSc = C::kScores;
  constexpr int kDmaIter = 2 * C::kDmaPerWave;   // direct loads a wave issues per iteration
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];
  char* const kbase = smem;                       // P2 ring
  char* const vbase = smem + C::kKRing;           // V ring
  char* const vsink = vbase + C::kVRing;
  int* const flags = reinterpret_cast<int*>(vsink + C::kVBlock);

  const int T = a.T;
  const int nq = (T + kBM - 1) / kBM;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;                       // query (column) within the wave
  const int hf = lane >> 5;                       // lane half
  const float k2 = hp.scale * kLog2e;             // raw dot -> log2-domain evidence

  // A operand of the row-sum MFMA (16x16x32, the weights as B operand): with
  // ones where lane bits 2 and 4 agree, lane l's result registers hold the
  // sum over both lane halves of query l % 32, i.e. its own row sum.
  bf16x8 sel;
  {
    const __bf16 v = (((lane >> 2) ^ (lane >> 4)) & 1) ? (__bf16)0.0f : (__bf16)1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = v;
  }

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
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  __bf16* Y = static_cast<__bf16*>(a.Y) + head;
  const auto rY = rsrc(Y, head_bytes);

  const int q0 = qt * kBM;
  const int qrow = q0 + wave * 32 + lq;           // may be >= T: loads give 0, stores drop
  // Iterations: 64-key tiles up to the tile's last row.
  const int kend = min(q0 + kBM, T) - 1;
  const int J = kend / kBN + 1;
  // The wave's diagonal 32-key block (-1: all its rows lie past T).
  const int dblk = q0 + wave * 32 < T ? q0 / 32 + wave : -1;
  const float inv_tau = hp.inv_tau[h];

  // Staging: wave w moves blocks k = w + 8 u of a P2 tile (row layout) and
  // of a V tile (transposed layout). P2 tiles >= J get an empty descriptor
  // (the loads still issue and write zeros but move no data); V tiles >= J
  // go to the sink block, so the ring keeps the last real ones.
  const int hb = (int)head_bytes;
  int dma_koff[C::kDmaPerWave], dma_voff[C::kDmaPerWave];
#pragma unroll
  for (int u = 0; u < C::kDmaPerWave; ++u) {
    const int k = wave + kWaves * u;
    dma_koff[u] = C::template row_src_real<DR>(k, lane);
    dma_voff[u] = C::template tr_src_real<DR>(k, lane);
  }
  auto dma_k = [&](int t, int slot) {
    const auto rs = rsrc_words(P2 + (size_t)t * kBN * DR, t < J ? hb - t * kBN * DR * 2 : 0);
    char* s = kbase + slot * C::kKBytes;
#pragma unroll
    for (int u = 0; u < C::kDmaPerWave; ++u) dma16(rs, s + (wave + kWaves * u) * C::kKBlock, dma_koff[u]);
  };
  auto dma_v = [&](int t) {
    const auto rs = rsrc_words(V + (size_t)t * kBN * DR, t < J ? hb - t * kBN * DR * 2 : 0);
    char* s = vbase + (t & (kVSlots - 1)) * C::kVBytes;
#pragma unroll
    for (int u = 0; u < C::kDmaPerWave; ++u)
      dma16(rs, t < J ? s + (wave + kWaves * u) * C::kVBlock : vsink, dma_voff[u]);
  };

  // Lane read bases of the P2 row layout and the transposed V reads, formed
  // once per use in a register (opaque to the optimiser), so every operand
  // read is that register plus an immediate.
  const int koff = C::row_base(lane);
  const int voff_even = C::tr_base(lane, false);
  const int voff_odd = C::tr_base(lane, true);
  auto kslot = [&](int t) -> const char* {
    unsigned off = (unsigned)((t & (kKSlots - 1)) * C::kKBytes + koff);
    asm volatile("" : "+v"(off));
    return smem + off;
  };
  auto vslot = [&](int t) -> VBase {
    const unsigned slot = (unsigned)(vbase - smem) + (unsigned)((t & (kVSlots - 1)) * C::kVBytes);
    unsigned e = slot + voff_even, o = slot + voff_odd;
    asm volatile("" : "+v"(e), "+v"(o));
    return VBase{smem + e, smem + o};
  };

  // Operand of step ii of a block: evidence k-step ii / 2 (even ii) of block
  // kbE of a P2 tile, or transport MFMA ii / 2 (odd ii) of block kbT of a V
  // tile.
  auto operand = [&](int ii, const char* kt, int kbE, const VBase& vt, int kbT) -> bf16x8 {
    if ((ii & 1) == 0) return *reinterpret_cast<const bf16x8*>(kt + C::k_imm(kbE, ii >> 1));
    return v_operand<D>(vt, kbT * 2 * C::kDb + (ii >> 1));
  };

  bf16x8 ring[4];                                 // step i reads ring[i % 4]
  f32x16 o[C::kDb];
  f32x4 l16;
  float lsum, dself, m2 = 0.0f;

  // One block step: evidence of block kbE of tile kt into sE, weights of sW
  // into pW, transport of block kbT of tile vt with pT; the last two steps
  // read the first operands of the next step (tiles ktn / vtn, blocks kbEn /
  // kbTn).
  auto step = [&](auto kind, f32x16& sE, const f32x16& sW, u32x4 (&pW)[2], const u32x4 (&pT)[2],
                  const char* kt, int kbE, const VBase& vt, int kbT, const char* ktn, int kbEn,
                  const VBase& vtn, int kbTn) __attribute__((always_inline)) {
    using K = decltype(kind);
    float tv[16];
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (K::W == kWDiag) dself = diag_entry(sW, hf, lq);
    // Weight of score n in two stages: tv = 1 / (1 + 2^-a), then
    // w = 2^(a tv - m2), masked on the diagonal block, packed in pairs.
    auto front = [&](int n) {
      const float an = kLse ? sW[n] * k2 : sW[n];
      tv[n] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-an));
    };
    auto back = [&](int n) {
      const float an = kLse ? sW[n] * k2 : sW[n];
      float w = __builtin_amdgcn_exp2f(an * tv[n] - m2);
      if constexpr (K::W == kWDiag) w = key_of(n, hf) < lq ? w : 0.0f;
      if constexpr (kLse) acc[n & 3] += w;
      if (n & 1) pW[n >> 3][(n & 7) >> 1] = pack_bf16(tv[n - 1], w);
      else tv[n] = w;
    };
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
      const int ip = i + 2;
      ring[ip & 3] = ip < kNS ? operand(ip, kt, kbE, vt, kbT) : operand(ip - kNS, ktn, kbEn, vtn, kbTn);
      if ((i & 1) == 0) {
        if constexpr (K::E) {
          const int ds = i >> 1;
          if (ds == 0) {
            const f32x16 zero = {};
            sE = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i & 3], qf[0], zero, 0, 0, 0);
          } else {
            sE = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i & 3], qf[ds], sE, 0, 0, 0);
          }
        }
      } else {
        if constexpr (K::T) {
          const int k = i >> 1, ks = k / C::kDb, db = k % C::kDb;
          const bf16x8 w = __builtin_bit_cast(bf16x8, pT[ks]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i & 3], w, o[db], 0, 0, 0);
          if constexpr (!kLse) {
            if (db == C::kDb - 1) l16 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, w, l16, 0, 0, 0);
          }
        }
      }
      if constexpr (K::W != kWOff) {
        if (i >= 1) {
#pragma unroll
          for (int n = (i - 1) * kSc; n < i * kSc; ++n) back(n);
        }
#pragma unroll
        for (int n = i * kSc; n < (i + 1) * kSc; ++n) front(n);
        if (i == kNS - 1) {
#pragma unroll
          for (int n = i * kSc; n < 16; ++n) back(n);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kLse && K::W != kWOff) lsum += (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  using SFull = StepKind<true, kWFull, true>;

  // Iteration end: wait for the previous iteration's direct loads (vector
  // memory operations complete in order, so vmcnt <= this iteration's count
  // suffices) and for every LDS read but the next iteration's first operands,
  // then meet the other waves.
  auto finish = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    wait_vm_lgkm<kDmaIter, 3>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int pass = 0;; ++pass) {
    // Prologue: P2 tiles 0..3 and V tiles 0..2 into their slots.
#pragma unroll
    for (int t = 0; t < 4; ++t) dma_k(t, t);
#pragma unroll
    for (int t = 0; t < 3; ++t) dma_v(t);
    wait_vm_lgkm<0, 15>();
    __syncthreads();
    if (!kLse && pass == 0) {
      // Scale the query rows by log2 e / sqrt(d_h) (bf16, round to nearest even).
#pragma unroll
      for (int ds = 0; ds < C::kDs; ++ds)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)((float)qf[ds][e] * k2);
    }
#pragma unroll
    for (int db = 0; db < C::kDb; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    l16 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lsum = 0.0f;
    dself = 0.0f;

    // Block roles rotate over two block steps per iteration:
    //   step 1: E(2j+2) -> sA, W(2j+1) from sB -> pA, T(2j) with pB;
    //   step 2: E(2j+3) -> sB, W(2j+2) from sA -> pB, T(2j+1) with pA.
    f32x16 sA, sB;
    u32x4 pA[2], pB[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[r] = sB[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pA[ks] = pB[ks] = u32x4{0u, 0u, 0u, 0u};
    {
      // E(0) -> sA, then the pre-step: E(1) -> sB, W(0) from sA -> pB.
      const char* k0 = kslot(0);
      if (dblk >= 0) sA = evidence_block<D>(k0, 0, qf);
      const VBase v0 = vslot(0);
      ring[0] = operand(0, k0, 1, v0, 0);
      ring[1] = operand(1, k0, 1, v0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const char* k1 = kslot(1);
      if (dblk >= 1) {
        step(StepKind<true, kWFull, false>{}, sB, sA, pB, pA, k0, 1, v0, 0, k1, 0, v0, 0);
      } else if (dblk == 0) {
        step(StepKind<false, kWDiag, false>{}, sB, sA, pB, pA, k0, 1, v0, 0, k1, 0, v0, 0);
      }
      // Iteration 0 loads P2 tile 4 into slot 0, which E(0) and the pre-step
      // read: every wave must be done with it first (all LDS reads but the
      // next three operands complete, then meet).
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      wait_vm_lgkm<63, 3>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }

    // Iteration j reads P2 tile j+1 and V tile j (and, in its last two
    // steps, the first operands of P2 tile j+2 and V tile j+1); it issues the
    // direct loads of P2 tile j+4 into the slot of tile j and of V tile j+3
    // into the slot of tile j-1, both last read in iteration j-1. The barrier
    // at its end publishes the tiles loaded in iteration j-1.
    // A wave's steady iterations are those with 2j+3 <= dblk (every block
    // role full; E(dblk) is an ordinary evidence block).
    const int jsteady = dblk >= 3 ? min(J, (dblk - 3) / 2 + 1) : 0;
    int j = 0;
    for (; j < jsteady; ++j) {
      dma_k(j + 4, j & (kKSlots - 1));
      dma_v(j + 3);
      const char* ka = kslot(j + 1);
      const char* kn = kslot(j + 2);
      const VBase va = vslot(j);
      const VBase vn = vslot(j + 1);
      step(SFull{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
      step(SFull{}, sB, sA, pB, pA, ka, 1, va, 1, kn, 0, vn, 0);
      finish();
    }
    for (; j < J; ++j) {
      dma_k(j + 4, j & (kKSlots - 1));
      dma_v(j + 3);
      const char* ka = kslot(j + 1);
      const char* kn = kslot(j + 2);
      const VBase va = vslot(j);
      const VBase vn = vslot(j + 1);
      const int r = dblk - 2 * j;                // the diagonal block relative to this tile
      if (r >= 3) {
        step(SFull{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
        step(SFull{}, sB, sA, pB, pA, ka, 1, va, 1, kn, 0, vn, 0);
      } else if (r == 2) {
        step(SFull{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
        step(StepKind<false, kWDiag, true>{}, sB, sA, pB, pA, ka, 1, va, 1, kn, 0, vn, 0);
      } else if (r == 1) {
        step(StepKind<false, kWDiag, true>{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
        step(StepKind<false, kWOff, true>{}, sB, sA, pB, pA, ka, 1, va, 1, kn, 0, vn, 0);
      } else if (r == 0) {
        step(StepKind<false, kWOff, true>{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
      }
      finish();
    }
    // The last iterations' direct loads (of tiles past the end) must land
    // before the ring is reused.
    wait_vm_lgkm<0, 15>();

    // Exactness of the fixed offset: every row sum below 2^100 and O finite.
    const float lrow = kLse ? lane_pair_sum(lsum) : l16[0];
    float omax = 0.0f;
#pragma unroll
    for (int db = 0; db < C::kDb; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) omax = fmaxf(omax, fabsf(o[db][r]));
    const bool ok = lrow <= kFinite && omax < INFINITY;
    const bool wave_bad = __any(!ok);
    if (lane == 0) flags[wave] = wave_bad ? 1 : 0;
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any_bad |= flags[w];
    any_bad = __builtin_amdgcn_readfirstlane(any_bad);
    __syncthreads();
    if (!any_bad || pass == 1) break;

    // Redo: an evidence-only pass over the history finds each row's maximum
    // a (the first row has none: its offset stays 0).
    float amax = -INFINITY;
    for (int t = 0; t < J; ++t) {
      dma_k(t, 0);
      wait_vm_lgkm<0, 15>();
      __syncthreads();
      const char* k0 = kslot(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int b = 2 * t + kb;
        if (b < dblk) amax = fmaxf(amax, block_max<false>(evidence_block<D>(k0, kb, qf), hf, lq));
        else if (b == dblk) amax = fmaxf(amax, block_max<true>(evidence_block<D>(k0, kb, qf), hf, lq));
      }
      wait_vm_lgkm<63, 0>();
      __syncthreads();
    }
    amax = lane_pair_max(amax);
    m2 = fmaxf(kLse ? amax * k2 : amax, 0.0f);
  }

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
  if (nqt >= 0) load_q(nqt, nbh);
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue -------------------------------------------------------------
  const float lrow = kLse ? lane_pair_sum(lsum) : l16[0];
  const float uii = lane_pair_sum(dself) * (kLse ? hp.scale : kLn2);
  const float S = sigmoid_f32(uii * inv_tau);
  const RowCombine c(S, m2 * kLn2, lrow, hp.lambda * logf((float)(qrow + 1)));
  if (kLse && hf == 0 && qrow < T) a.lse[(size_t)bh * T + qrow] = c.lse;
  const int roff = qrow * (DR * 2) + hf * 8;
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

template <int D, int DR>
hipError_t launch_typed(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  const int nq = (a.T + kBM - 1) / kBM;
  const long long nwork = (long long)((nq + 1) / 2) * a.B * a.H;
  if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
  // One persistent work-group per compute unit (the LDS rings admit one).
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const long long grid = nwork < n_cu ? nwork : n_cu;
  if (a.lse != nullptr) {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, DR, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, hp);
  } else {
    hipLaunchKernelGGL((fwd_mfma_kernel<D, DR, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, hp);
  }
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
    case 64: return launch_typed<64, 64>(a, hp, s);
    case 80: return launch_typed<128, 80>(a, hp, s);
    case 128: return launch_typed<128, 128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

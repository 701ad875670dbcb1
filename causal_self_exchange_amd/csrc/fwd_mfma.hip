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
// previous one); operand reads run two MFMAs ahead, also across tiles. Two
// block steps make one iteration over a 64-key tile.
//
// The waves do not meet at a barrier per iteration: each one counts its
// finished iterations in an LDS counter, and a wave waits only where it
// refills the ring, between its two block steps, until every wave has
// finished the previous iteration (so the slots it overwrites are no longer
// read and the tiles it reads next have landed). The waves of a SIMD may thus
// drift apart by up to an iteration and a half and keep both issuing.
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
  // needed (so the ring keeps the work-group's own rows), + 8 wave flags and
  // the iteration counter.
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

// Lane index read afresh (v_mbcnt) wherever it is used: the optimiser cannot
// merge the reads, so no lane-derived value has to stay live (or be spilled)
// across the key loop just to be used again after it.
__device__ __forceinline__ int lane_now() {
  unsigned l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return (int)l;
}

// LDS counter increment by lane 0 of the calling wave (exec narrowed to that
// lane inside the statement, so no branch splits the caller's code). The
// s_nop separates the VALU write of the data VGPR from the LDS instruction
// that reads it, as the compiler does for its own code (its hazard checks do
// not look inside inline assembly).
__device__ __forceinline__ void lds_count_up(unsigned* p) {
  const unsigned addr = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned*)p;
  unsigned long long save;
  unsigned one;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "v_mov_b32 %1, 1\n\t"
      "s_nop 1\n\t"
      "ds_add_u32 %2, %1\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(save), "=&v"(one)
      : "v"(addr)
      : "memory");
}

// Wait until the LDS counter *p has reached `want` (wrapping compare),
// polling with a short sleep between reads. The loop is one assembly
// statement: the compiler sees no basic-block boundary and moves no code into
// or across it. Its hazard checks do not look inside the statement either:
// v_readfirstlane reading a VGPR that the previous VALU instruction wrote
// needs a wait state on this architecture (without it the read can return
// the VGPR's older value), so the read is preceded by s_nop although here the
// VGPR comes from an LDS load. (An SALU read of an SGPR that v_readfirstlane
// wrote needs none.)
__device__ __forceinline__ void lds_wait_count(const unsigned* p, unsigned want) {
  const unsigned addr = (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned*)p;
  unsigned v, d;
  asm volatile(
      "1:\n\t"
      "ds_read_b32 %0, %2\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 1\n\t"
      "v_readfirstlane_b32 %1, %0\n\t"
      "s_sub_u32 %1, %1, %3\n\t"
      "s_cmp_lt_i32 %1, 0\n\t"
      "s_cbranch_scc0 2f\n\t"
      "s_sleep 1\n\t"
      "s_branch 1b\n"
      "2:"
      : "=&v"(v), "=&s"(d)
      : "v"(addr), "s"(want)
      : "memory", "scc");
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
// the rows' real head size in memory (32 and 48 run on the 64 layout and 80
// on the 128 layout, the chunks past DR held at zero, so evidence and
// transport are exact and the padded output rows are not stored).
// kRope: P1 is rotated (rotary position encoding, interleaved or half-split
// pairs) after each query tile's rows are loaded, as the pre-step would have
// rotated it (same angles, fp32 rotation, one bf16 rounding).
template <int D, int DR, bool kLse, bool kRope>
__device__ __forceinline__ void fwd_body(const FwdArgs& a, const HeadParams& hp, const RopeParams& rp) {
  static_assert(DR % 16 == 0 && DR <= D && DR >= 32, "real head size within the layout");
  using C = Cfg<D>;
  constexpr int kNS = C::kSteps;
  constexpr int kSc = C::kScores;
  constexpr int kDmaIter = 2 * C::kDmaPerWave;   // direct loads a wave issues per iteration
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];
  char* const kbase = smem;                       // P2 ring
  char* const vbase = smem + C::kKRing;           // V ring
  char* const vsink = vbase + C::kVRing;
  int* const flags = reinterpret_cast<int*>(vsink + C::kVBlock);
  // done_iters counts the iterations the waves have finished (one increment
  // per wave and iteration, the pre-step of a tile included); `arrived` is its
  // value once every wave has finished what this wave has. Neither is ever
  // reset: they wrap, and only differences are compared.
  unsigned* const done_iters = reinterpret_cast<unsigned*>(flags + kWaves);
  unsigned arrived = 0;

  const int T = a.T;
  const int nq = (T + kBM - 1) / kBM;
  const int tid = threadIdx.x;
  if (tid == 0) *done_iters = 0u;   // ordered before any use by the first tile's barrier
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Lane l holds query (column) lq = l % 32 of the wave's rows, lane half
  // hf = l / 32; both are formed from lane_now() where they are used.
  const float k2 = hp.scale * kLog2e;             // raw dot -> log2-domain evidence

  // A operand of the row-sum MFMA (16x16x32, the weights as B operand): with
  // ones where lane bits 2 and 4 agree, lane l's result registers hold the
  // sum over both lane halves of query l % 32, i.e. its own row sum.
  bf16x8 sel;
  {
    const int lane = lane_now();
    const __bf16 v = (((lane >> 2) ^ (lane >> 4)) & 1) ? (__bf16)0.0f : (__bf16)1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = v;
  }

  // P1 rows of a query tile as the evidence MFMA's B operand: lane holds
  // p1[qrow][16 ds + 8 hf + 0..7]. They are loaded at the end of the previous
  // tile, so their latency overlaps that of the next tile's first key tiles
  // (loading them earlier would hold them through the epilogue, where any
  // wait on vector memory would also wait for them).
  bf16x8 qf[C::kDs];
  auto load_q = [&](int qt, int bh) __attribute__((always_inline)) {
    const auto rP1 = rsrc(static_cast<const __bf16*>(a.P1) + (size_t)bh * (size_t)T * DR, (long long)T * DR * 2);
    const int lane = lane_now();
    const int qoff = (qt * kBM + wave * 32 + (lane & 31)) * (DR * 2) + (lane >> 5) * 16;
#pragma unroll
    for (int ds = 0; ds < C::kDs; ++ds) {
      // k-steps past DR / 16 cover padded columns: out-of-range offsets read 0.
      const int o = ds < DR / 16 ? qoff + ds * 32 : kOutOfRange;
      qf[ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP1, o, 0, 0));
    }
  };

  // Rotate the loaded query rows of tile qt of head bh (kRope). The lane
  // holds row q0 + 32 wave + lane % 32 at columns 16 ds + 8 (lane / 32) + e:
  // interleaved pair k = (2k, 2k+1) lies in one 8-element chunk; half-split
  // pair k = (k, k + DR/2) lies in chunks ds and ds + DR/32 of the same lane.
  auto rope_q = [&](int qt, int bh) __attribute__((always_inline)) {
    if constexpr (kRope) {
      const int lane = lane_now();
      const int hf = lane >> 5;
      const int row = qt * kBM + wave * 32 + (lane & 31);
      const long long p0 = rp.pos0 ? (long long)rp.pos0[bh / a.H] : 0;
      const double pos = (double)(p0 + row);
      // (x, y) -> (x cos - y sin, x sin + y cos), in fp32, rounded to bf16
      auto turn = [&](float u, float v, int k, __bf16* out) __attribute__((always_inline)) {
        float sn, cs;
        sincos_of(pos * rp.inv_freq[k], &sn, &cs);
        out[0] = (__bf16)fmaf(u, cs, -v * sn);
        out[1] = (__bf16)fmaf(u, sn, v * cs);
      };
      if (rp.rope == 1) {
#pragma unroll
        for (int ds = 0; ds < DR / 16; ++ds)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            __bf16 r[2];
            turn((float)qf[ds][2 * e], (float)qf[ds][2 * e + 1], 8 * ds + 4 * hf + e, r);
            qf[ds][2 * e] = r[0];
            qf[ds][2 * e + 1] = r[1];
          }
      } else if constexpr (DR % 32 == 0) {
#pragma unroll
        for (int ds = 0; ds < DR / 32; ++ds)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            __bf16 r[2];
            turn((float)qf[ds][e], (float)qf[ds + DR / 32][e], 16 * ds + 8 * hf + e, r);
            qf[ds][e] = r[0];
            qf[ds + DR / 32][e] = r[1];
          }
      }
    }
  };

  // Scale the query rows by log2 e / sqrt(d_h) (bf16, round to nearest even).
  auto prescale_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ds = 0; ds < C::kDs; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)((float)qf[ds][e] * k2);
  };

  // One query tile (256 rows) of one head, start to finish; then, when nqt >=
  // 0, the P1 rows of query tile nqt of head nbh are loaded.
  auto run_tile = [&](int qt, int bh, int nqt, int nbh) __attribute__((always_inline)) {
  const int h = bh % a.H;
  const size_t head = (size_t)bh * (size_t)T * DR;
  const long long head_bytes = (long long)T * DR * 2;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  __bf16* Y = static_cast<__bf16*>(a.Y) + head;
  const auto rY = rsrc(Y, head_bytes);

  const int q0 = qt * kBM;
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
  const int lane = lane_now();
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
    int lq = 0, hf = 0;
    if constexpr (K::W == kWDiag) {
      const int ln = lane_now();
      lq = ln & 31;
      hf = ln >> 5;
      dself = diag_entry(sW, hf, lq);
    }
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

  // Ring hand-over without a barrier (done_iters / arrived above).
  // An iteration ends once the wave's direct loads of the previous iteration
  // have landed (vector memory operations complete in order, so vmcnt <= this
  // iteration's count suffices) and all its LDS reads but the next
  // iteration's first operands are done.
  auto arrive = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    wait_vm_lgkm<kDmaIter, 3>();
    lds_count_up(done_iters);
    arrived += kWaves;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Iteration j, between its block steps: once every wave has finished
  // iteration j - 1 or the pre-step (so it read the slots of P2 tile j and V tile j - 1 for
  // the last time, and its loads of P2 tile j + 3 and V tile j + 2 landed),
  // load P2 tile j + 4 and V tile j + 3 into those slots. The slowest wave
  // never waits here, so the wait always ends.
  auto refill = [&](int jj) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    lds_wait_count(done_iters, arrived);
    dma_k(jj + 4, jj & (kKSlots - 1));
    dma_v(jj + 3);
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int pass = 0;; ++pass) {
    // Prologue: P2 tiles 0..3 and V tiles 0..2 into their slots, in the order
    // they are read: P2 0, 1 and V 0 (the pre-step), P2 2 and V 1 (the end of
    // iteration 0), P2 3 and V 2 (the end of iteration 1). Only the first
    // group is waited for here; the pre-step's arrival certifies the second
    // and iteration 0's the third (vector memory operations complete in
    // order, and each arrival waits for all but its last kDmaIter).
    dma_k(0, 0);
    dma_k(1, 1);
    dma_v(0);
    dma_k(2, 2);
    dma_v(1);
    dma_k(3, 3);
    dma_v(2);
    wait_vm_lgkm<4 * C::kDmaPerWave, 15>();
    __syncthreads();
    if (pass == 0) {                        // the redo transforms its own reload
      rope_q(qt, bh);
      if (!kLse) prescale_q();
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
      // read: the pre-step counts as an iteration.
      arrive();
    }

    // Iteration j reads P2 tile j+1 and V tile j (and, in its last two
    // steps, the first operands of P2 tile j+2 and V tile j+1); between its
    // block steps it loads P2 tile j+4 into the slot of tile j and V tile j+3
    // into the slot of tile j-1, both last read in iteration j-1.
    // A wave's steady iterations are those with 2j+3 <= dblk (every block
    // role full; E(dblk) is an ordinary evidence block).
    const int jsteady = dblk >= 3 ? min(J, (dblk - 3) / 2 + 1) : 0;
    int j = 0;
    for (; j < jsteady; ++j) {
      const char* ka = kslot(j + 1);
      const char* kn = kslot(j + 2);
      const VBase va = vslot(j);
      const VBase vn = vslot(j + 1);
      step(SFull{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
      refill(j);
      step(SFull{}, sB, sA, pB, pA, ka, 1, va, 1, kn, 0, vn, 0);
      arrive();
    }
    // The diagonal block relative to the next iteration: r = dblk - 2j is 1
    // or 2 after the steady iterations (the diagonal block's tile dblk / 2 is
    // at most J - 1), dblk itself when there were none, negative for a wave
    // whose rows all lie past T. What is left is straight-line: at most two
    // iterations with work, then iterations that only move tiles.
    const int r = dblk - 2 * j;
    if (r == 2) {
      {
        const char* ka = kslot(j + 1);
        const VBase va = vslot(j);
        step(SFull{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
        refill(j);
        step(StepKind<false, kWDiag, true>{}, sB, sA, pB, pA, ka, 1, va, 1, kslot(j + 2), 0, vslot(j + 1), 0);
        arrive();
        ++j;
      }
      {
        const char* ka = kslot(j + 1);
        const VBase va = vslot(j);
        step(StepKind<false, kWOff, true>{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
        refill(j);
        arrive();
        ++j;
      }
    } else if (r == 1) {
      const char* ka = kslot(j + 1);
      const VBase va = vslot(j);
      step(StepKind<false, kWDiag, true>{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
      refill(j);
      step(StepKind<false, kWOff, true>{}, sB, sA, pB, pA, ka, 1, va, 1, kslot(j + 2), 0, vslot(j + 1), 0);
      arrive();
      ++j;
    } else if (r == 0) {
      const char* ka = kslot(j + 1);
      const VBase va = vslot(j);
      step(StepKind<false, kWOff, true>{}, sA, sB, pA, pB, ka, 0, va, 0, ka, 1, va, 1);
      refill(j);
      arrive();
      ++j;
    }
    for (; j < J; ++j) {
      refill(j);
      arrive();
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
    if (lane_now() == 0) flags[wave] = wave_bad ? 1 : 0;
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any_bad |= flags[w];
    any_bad = __builtin_amdgcn_readfirstlane(any_bad);
    __syncthreads();
    if (!any_bad || pass == 1) break;

    // Redo: an evidence-only pass over the history finds each row's maximum
    // a (the first row has none: its offset stays 0). The P1 rows are loaded
    // (and scaled) again here rather than kept live through the end of the
    // scan, which would hold their registers in every tile.
    load_q(qt, bh);
    wait_vm_lgkm<0, 15>();
    rope_q(qt, bh);
    if (!kLse) prescale_q();
    float amax = -INFINITY;
    const int lq = lane_now() & 31, hf = lane_now() >> 5;
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
  const int lq = lane_now() & 31, hf = lane_now() >> 5;
  const int qrow = q0 + wave * 32 + lq;           // may be >= T: the stores drop it
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

  // ---- epilogue -------------------------------------------------------------
  const float lrow = kLse ? lane_pair_sum(lsum) : l16[0];
  const float uii = lane_pair_sum(dself) * (kLse ? hp.scale : kLn2);
  const float S = sigmoid_f32(uii * inv_tau);
  const RowCombine c(S, m2 * kLn2, lrow, hp.lambda * logf((float)(qrow + 1)));
  if (kLse && hf == 0 && qrow < T) a.lse[(size_t)bh * T + qrow] = c.lse;
  // The rows of Y pass through LDS, so that each store writes whole rows:
  // the P2 ring is free once every wave has left the key loop, and each wave
  // uses its own part of it (32 rows of 2 D + 16 bytes; the 16 bytes of
  // padding spread a column's rows over the banks).
  constexpr int kYStride = 2 * D + 16;
  static_assert(kWaves * 32 * kYStride <= C::kKRing, "Y staging fits in the P2 ring");
  char* const ystage = kbase + wave * 32 * kYStride;
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      if (32 * db + 8 * g4 >= DR) continue;      // padded columns
      bf16x4 yy;
#pragma unroll
      for (int e = 0; e < 4; ++e) yy[e] = (__bf16)(c.w_self * (float)vv[db][g4][e] + c.w_hist * o[db][4 * g4 + e]);
      *reinterpret_cast<bf16x4*>(ystage + lq * kYStride + 2 * (32 * db + 8 * g4 + 4 * hf)) = yy;
    }
  }
  // A wave reads back only what its own lanes wrote (its LDS operations
  // complete in order; the wave barrier only marks the dependence between
  // lanes): 16-byte chunk ch of rows 64 / (D / 8) apart per store, so one
  // store covers 64 / (D / 8) whole rows; chunks past DR are not stored, nor
  // rows >= T (outside the descriptor's range).
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int kC = D / 8;
    constexpr int kRows = 64 / kC;
    const int ln = lane_now();
    const int ch = ln % kC, rs = ln / kC;
#pragma unroll
    for (int i = 0; i < 32 / kRows; ++i) {
      const int rr = i * kRows + rs;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ystage + rr * kYStride + 16 * ch);
      const int off = ch < DR / 8 ? (q0 + wave * 32 + rr) * (DR * 2) + 16 * ch : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b128(v, rY, off, 0, 0);
    }
  }
  // Every wave is done with both rings (V_i, Y staging) before the next
  // tile's loads refill them.
  wait_vm_lgkm<63, 0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (nqt >= 0) load_q(nqt, nbh);
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

template <int D, int DR, bool kLse>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_kernel(FwdArgs a, HeadParams hp) {
  const RopeParams none{};
  fwd_body<D, DR, kLse, false>(a, hp, none);
}

template <int D, int DR, bool kLse>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_rope_kernel(FwdArgs a, HeadParams hp, RopeParams rp) {
  fwd_body<D, DR, kLse, true>(a, hp, rp);
}

template <int D, int DR>
hipError_t launch_typed(const FwdArgs& a, const HeadParams& hp, hipStream_t s, const RopeParams* rp) {
  const int nq = (a.T + kBM - 1) / kBM;
  const long long nwork = (long long)((nq + 1) / 2) * a.B * a.H;
  if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
  // One persistent work-group per compute unit (the LDS rings admit one).
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const long long grid = nwork < n_cu ? nwork : n_cu;
  if (rp != nullptr) {
    if (a.lse != nullptr) {
      hipLaunchKernelGGL((fwd_mfma_rope_kernel<D, DR, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, hp, *rp);
    } else {
      hipLaunchKernelGGL((fwd_mfma_rope_kernel<D, DR, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, hp, *rp);
    }
  } else if (a.lse != nullptr) {
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
  return (d_h == 32 || d_h == 48 || d_h == 64 || d_h == 80 || d_h == 128) && ((long long)T + kBM) * d_h * 2 < 0x7fffffffLL;
}

bool fwd_mfma_rope_fusable(int d_h, int rope) {
  return (d_h == 32 || d_h == 48 || d_h == 64 || d_h == 80 || d_h == 128) && (rope == 1 || (rope == 2 && d_h % 32 == 0));
}

hipError_t launch_fwd_mfma_bf16(const FwdArgs& a, const HeadParams& hp, hipStream_t s, const RopeParams* rp) {
  if (rp != nullptr && !fwd_mfma_rope_fusable(a.d_h, rp->rope)) return hipErrorInvalidValue;
  switch (a.d_h) {
    case 32: return launch_typed<64, 32>(a, hp, s, rp);
    case 48: return launch_typed<64, 48>(a, hp, s, rp);
    case 64: return launch_typed<64, 64>(a, hp, s, rp);
    case 80: return launch_typed<128, 80>(a, hp, s, rp);
    case 128: return launch_typed<128, 128>(a, hp, s, rp);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

// bf16 MFMA FlashRelation forward for gfx950 ("Ask Self, Ask Others: Relation
// Is All You Need", Sec. 5.1, Eq. (12)-(14); App. A.3).
//
// Work-group = 4 waves = 128 query rows of one (b, h); each wave owns 32 rows.
// Key tiles of 64 rows of P2 and V are staged through LDS (double-buffered,
// XOR-swizzled 16-byte chunks, coalesced 16-byte global loads) and shared by
// the 4 waves. Per tile and wave:
//   evidence  S^T[key][query] = P2 . P1^T  on v_mfma_f32_32x32x16_bf16; the
//             transposed product puts one query per lane, so a row's 64
//             scores sit in one lane pair (l, l^32);
//   roles     diagonal tile: keys j >= i of the row are removed (Self is not
//             part of the Exchange scan); Exchange E = SiLU(U) in registers;
//   scan      running stabiliser m (log2 domain) starting at 0, which is
//             valid because SiLU(u) <= max(u, 0) and SiLU >= -0.2785, so the
//             largest weight of a non-empty history is >= e^-0.2785;
//             m moves only when the tile maximum exceeds it by > 8 (lazy
//             rescaling); weights p = exp(E - m) go to bf16;
//   transport O^T[d][query] += V^T . P^T on the same MFMA; V^T operands come
//             straight from the row-major LDS tile via ds_read_b64_tr_b16.
// Epilogue: Self entry S_i = sigmoid(U_ii / tau) from p1_i . p2_i in fp32,
// count term lambda log i, and the branch-free Self/Exchange combination;
// the first row gets Y_1 = V_1 exactly.
//
// Causal tile skip: a work-group scans only key tiles left of its last row;
// inside, a wave skips 32-key blocks right of its own diagonal block.
// Grid order: heaviest query tiles first, and when B*H is a multiple of 8,
// all query tiles of one head go to one XCD (work-groups are dealt to the
// 8 XCDs round-robin), so the head's P2/V stay in that XCD's L2.
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;          // query rows per work-group
constexpr int kBN = 64;           // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;     // rescale only when the max grows by > 2^8

template <int D>
struct Lds {
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBN * kRowBytes;
  // XOR swizzle of the chunk index by row, chosen so that the 16-lane b128
  // reads of P2 rows, the 32-lane transposed b64 reads of V and the tile
  // writes each touch distinct banks.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
      return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
    }
  }
  __device__ static __forceinline__ int off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
};

__device__ __forceinline__ float lane_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ s16x4 lds_tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// (query tile, b*H + h) of this work-group: heaviest tiles first; one head's
// tiles on one XCD when the head count allows.
__device__ __forceinline__ void tile_of_block(int n, int nq, int BH, int& qt, int& bh) {
  if ((BH & 7) == 0) {
    const int per = BH >> 3;          // heads per XCD
    const int xcd = n & 7, loc = n >> 3;
    bh = xcd * per + loc % per;
    qt = nq - 1 - loc / per;
  } else {
    qt = nq - 1 - n / BH;
    bh = n % BH;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(FwdArgs a, HeadParams hp) {
  using L = Lds<D>;
  constexpr int kDs = D / 16;                    // k-steps of the evidence MFMA
  constexpr int kDb = D / 32;                    // 32-row blocks of O^T
  constexpr int kLoads = kBN * L::kChunks / kThreads;
  __shared__ __attribute__((aligned(16))) char smem[2][2][L::kTileBytes];   // [buf][P2|V]

  const int T = a.T;
  const int nq = (T + kBM - 1) / kBM;
  int qt, bh;
  tile_of_block(blockIdx.x, nq, a.B * a.H, qt, bh);
  const int h = bh % a.H;
  const size_t head = (size_t)bh * (size_t)T * D;
  const __bf16* P1 = static_cast<const __bf16*>(a.P1) + head;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  __bf16* Y = static_cast<__bf16*>(a.Y) + head;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;                      // query (column) within the wave
  const int hf = lane >> 5;                      // lane half
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + lq;
  const bool qvalid = qrow < T;

  // P1 rows as the evidence MFMA's B operand: lane holds p1[qrow][16 ds + 8 hf + 0..7].
  bf16x8 qf[kDs];
#pragma unroll
  for (int ds = 0; ds < kDs; ++ds) {
    if (qvalid) {
      qf[ds] = *reinterpret_cast<const bf16x8*>(P1 + (size_t)qrow * D + 16 * ds + 8 * hf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)0.0f;
    }
  }

  f32x16 o[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m2 = 0.0f;                               // stabiliser, log2 domain
  float lsum = 0.0f;                             // this lane's share of the row sum

  const float k2 = hp.scale * kLog2e;            // raw dot -> log2-domain evidence
  // Keys 0 .. kend-1 are history for some row of this tile.
  const int kend = min(q0 + kBM, T) - 1;
  const int ntiles = (kend + kBN - 1) / kBN;

  // Staging: thread loads chunk e = it * kThreads + tid of the tile.
  uint4 kreg[kLoads], vreg[kLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int e = it * kThreads + tid;
      const int row = e / L::kChunks, ch = e % L::kChunks;
      const int j = t * kBN + row;
      if (j < T) {
        kreg[it] = *reinterpret_cast<const uint4*>(P2 + (size_t)j * D + ch * 8);
        vreg[it] = *reinterpret_cast<const uint4*>(V + (size_t)j * D + ch * 8);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int e = it * kThreads + tid;
      const int row = e / L::kChunks, ch = e % L::kChunks;
      *reinterpret_cast<uint4*>(&smem[buf][0][L::off(row, ch)]) = kreg[it];
      *reinterpret_cast<uint4*>(&smem[buf][1][L::off(row, ch)]) = vreg[it];
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  // Lane-constant parts of the transposed V read: 16-lane group g, index i.
  const int tg = lane >> 4, ti = lane & 15;
  const int tr_row = 4 * (tg >> 1) + (ti >> 2);  // + 16 ks + 8 rd + 32 kb
  const int tr_col = 16 * (tg & 1) + 4 * (ti & 3);  // + 32 db

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const char* kb_lds = smem[buf][0];
    const char* vb_lds = smem[buf][1];

    // Status of the tile's two 32-key blocks for this wave.
    const int kbase0 = t * kBN;
    const bool act0 = kbase0 <= qw0, act1 = kbase0 + 32 <= qw0;
    if (act0) {
      const bool diag0 = kbase0 == qw0, diag1 = kbase0 + 32 == qw0;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
        if (kb == 1 && !act1) continue;
#pragma unroll
        for (int ds = 0; ds < kDs; ++ds) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb_lds + L::off(kb * 32 + lq, 2 * ds + hf));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[kb], 0, 0, 0);
        }
      }
      // Key of register r in a 32-key block, relative to the block: 8(r/4) + 4 hf + r%4.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool act = kb == 0 ? true : act1;
        const bool diag = kb == 0 ? diag0 : diag1;
        if (!act) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jr = 8 * (r >> 2) + 4 * hf + (r & 3);
          const float x = (diag && jr >= lq) ? -INFINITY : s[kb][r];
          mx = fmaxf(mx, x);
        }
      }
      mx = lane_pair_max(mx);
      const float mc2 = fmaxf(mx, 0.0f) * k2;
      const float mnew = mc2 > m2 + kLazy ? mc2 : m2;
      if (__any(mnew != m2)) {
        const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < kDb; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m2 = mnew;
      }
      // Exchange weights p = exp(SiLU(u) - m): with a = u log2 e,
      // SiLU(u) log2 e = a / (1 + 2^-a).
      bf16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool act = kb == 0 ? true : act1;
        const bool diag = kb == 0 ? diag0 : diag1;
        if (!act) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float av = s[kb][r] * k2;
          const float den = 1.0f + __builtin_amdgcn_exp2f(-av);
          float p = __builtin_amdgcn_exp2f(av * __builtin_amdgcn_rcpf(den) - m2);
          if (diag) {
            const int jr = 8 * (r >> 2) + 4 * hf + (r & 3);
            p = jr < lq ? p : 0.0f;
          }
          lsum += p;
          pf[kb][r >> 3][r & 7] = (__bf16)p;
        }
      }
      // Transport: O^T[d][q] += V^T[d][key] P^T[key][q].
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !act1) continue;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int row = kb * 32 + 16 * ks + tr_row;
#pragma unroll
          for (int db = 0; db < kDb; ++db) {
            const int col = 32 * db + tr_col;
            const int ch = col >> 3, half = (col >> 2) & 1;
            const s16x4 lo = lds_tr_read(vb_lds + L::off(row, ch) + 8 * half);
            const s16x4 hi = lds_tr_read(vb_lds + L::off(row + 8, ch) + 8 * half);
            bf16x8 vf;
            vf.lo = __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(4))), lo);
            vf.hi = __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(4))), hi);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][ks], o[db], 0, 0, 0);
          }
        }
      }
    }

    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  lsum = lane_pair_sum(lsum);
  float dself = 0.0f;
  if (qvalid) {
#pragma unroll
    for (int ds = 0; ds < kDs; ++ds) {
      const bf16x8 k2v = *reinterpret_cast<const bf16x8*>(P2 + (size_t)qrow * D + 16 * ds + 8 * hf);
#pragma unroll
      for (int e = 0; e < 8; ++e) dself = fmaf((float)qf[ds][e], (float)k2v[e], dself);
    }
  }
  dself = lane_pair_sum(dself);
  if (!qvalid) return;
  const float S = sigmoid_f32(dself * hp.scale * hp.inv_tau[h]);
  const RowCombine c(S, m2 * kLn2, lsum, hp.lambda * logf((float)(qrow + 1)));
  const __bf16* vrow = V + (size_t)qrow * D;
  __bf16* yrow = Y + (size_t)qrow * D;
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * hf;
      const uint2 vraw = *reinterpret_cast<const uint2*>(vrow + d0);
      const __bf16* vv = reinterpret_cast<const __bf16*>(&vraw);
      uint2 yraw;
      __bf16* yy = reinterpret_cast<__bf16*>(&yraw);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        yy[e] = (__bf16)(c.w_self * (float)vv[e] + c.w_hist * o[db][4 * g4 + e]);
      *reinterpret_cast<uint2*>(yrow + d0) = yraw;
    }
  }
}

template <int D>
hipError_t launch_typed(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  const int nq = (a.T + kBM - 1) / kBM;
  const long long blocks = (long long)nq * a.B * a.H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_mfma_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a, hp);
  return hipGetLastError();
}

}  // namespace

bool fwd_mfma_supported(int d_h) { return d_h == 64 || d_h == 128; }

hipError_t launch_fwd_mfma_bf16(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  switch (a.d_h) {
    case 64: return launch_typed<64>(a, hp, s);
    case 128: return launch_typed<128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

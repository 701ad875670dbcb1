// bf16 MFMA FlashRelation forward for gfx950 ("Ask Self, Ask Others: Relation
// Is All You Need", Sec. 5.1, Eq. (12)-(14); App. A.3).
//
// Work-group = 4 waves = 128 query rows of one (b, h); each wave owns 32 rows.
// Key tiles of 64 rows of P2 and V are staged through LDS (double-buffered,
// row pitch padded so every read address is a lane base plus an immediate,
// loads through buffer descriptors whose range check zero-fills rows >= T)
// and shared by the 4 waves. Per tile and wave:
//   evidence  S^T[key][query] = P2 . P1^T  on v_mfma_f32_32x32x16_bf16; the
//             transposed product puts one query per lane, so a row's 64
//             scores sit in one lane pair (l, l^32);
//   roles     only the diagonal tile removes keys j >= i of the row (Self is
//             not part of the Exchange scan); Exchange E = SiLU(U) in
//             registers; every other tile runs without any mask;
//   scan      running stabiliser m (log2 domain) starting at 0, which is
//             valid because SiLU(u) <= max(u, 0) and SiLU >= -0.2785, so the
//             largest weight of a non-empty history is >= e^-0.2785;
//             m moves only when the tile maximum exceeds it by > 8 (lazy
//             rescaling); weights p = exp(E - m) go to bf16 and the row sum
//             is accumulated from those bf16 weights with v_dot2;
//   transport O^T[d][query] += V^T . P^T on the same MFMA; V^T operands come
//             straight from the row-major LDS tile via ds_read_b64_tr_b16.
// Epilogue: Self entry S_i = sigmoid(U_ii / tau) from p1_i . p2_i in fp32,
// count term lambda log i, and the branch-free Self/Exchange combination;
// the first row gets Y_1 = V_1 exactly.
//
// Causal tile skip: a work-group scans only key tiles left of its last row;
// in the last two tiles a wave skips 32-key blocks right of its diagonal.
// Grid order: heaviest query tiles first; when B*H is a multiple of 8 the
// query tiles of one head run together on one XCD (work-groups are dealt to
// the 8 XCDs round-robin), so the head's P2/V stay in that XCD's L2.
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;          // query rows per work-group
constexpr int kBN = 64;           // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;     // rescale only when the max grows by > 2^8
constexpr int kBufFlags = 0x00020000;   // raw buffer descriptor word 3 (gfx9)

template <int D>
struct Cfg {
  static constexpr int kChunks = D / 8;              // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  // P2 rows: +16 B so 16 consecutive rows start in 16 different bank groups
  // (conflict-free 16-byte evidence-operand reads by 16 lanes).
  static constexpr int kPitchK = kRowBytes + 16;
  // V rows: +64 B so the transposed 8-byte reads of 4 rows x 64 B by 32 lanes
  // hit 32 different bank pairs.
  static constexpr int kPitchV = kRowBytes + 64;
  static constexpr int kKBytes = kBN * kPitchK;
  static constexpr int kVBytes = kBN * kPitchV;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kRowsPerPass = kThreads / kChunks;   // staging rows per pass
  static constexpr int kLoads = kBN / kRowsPerPass;
};

__device__ __forceinline__ float lane_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 lds_tr_read(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufFlags);
}

// (query tile, b*H + h) of this work-group: heaviest tiles first; when the
// head count allows, each XCD runs the query tiles of one head at a time, so
// that head's P2/V tiles stay in the XCD's L2.
__device__ __forceinline__ void tile_of_block(int n, int nq, int BH, int& qt, int& bh) {
  if ((BH & 7) == 0) {
    const int per = BH >> 3;          // heads per XCD
    const int xcd = n & 7, loc = n >> 3;
    bh = xcd * per + loc / nq;
    qt = nq - 1 - loc % nq;
  } else {
    qt = nq - 1 - n / BH;
    bh = n % BH;
  }
}

// Block modes of a 64-key tile for one wave (blocks kb0 = keys 0..31, kb1 = 32..63):
//   0: both blocks strictly left of the wave's rows (no mask);
//   1: kb0 full, kb1 is the wave's diagonal block;
//   2: kb0 is the diagonal block, kb1 lies to the right (skipped).
template <int D, int MODE>
__device__ __forceinline__ void tile_step(const char* kl, const char* vl, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&o)[D / 32], float& m2, float& lsum, float k2,
                                          int lq, int hf, int koff, int voff) {
  using C = Cfg<D>;
  constexpr int kDs = D / 16;
  constexpr int kDb = D / 32;
  constexpr int kBlocks = MODE == 2 ? 1 : 2;
  constexpr bool kDiag0 = MODE == 2;
  constexpr bool kDiag1 = MODE == 1;

  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < kBlocks; ++kb) {
#pragma unroll
    for (int ds = 0; ds < kDs; ++ds) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + koff + kb * 32 * C::kPitchK + ds * 32);
      if (ds == 0) {
        const f32x16 zero = {};
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], zero, 0, 0, 0);
      } else {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[kb], 0, 0, 0);
      }
    }
  }

  // Key of register r within a 32-key block: 8 (r / 4) + 4 hf + r % 4.
  // Four independent partial maxima keep the dependency chain short.
  float mxp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int kb = 0; kb < kBlocks; ++kb) {
    const bool diag = kb == 0 ? kDiag0 : kDiag1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[kb][r];
      if (diag) x = (8 * (r >> 2) + 4 * hf + (r & 3)) < lq ? x : -INFINITY;
      mxp[r & 3] = fmaxf(mxp[r & 3], x);
    }
  }
  float mx = lane_pair_max(fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3])));
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

  // Exchange weights p = exp(SiLU(u) - m) with a = u log2 e:
  // SiLU(u) log2 e = a / (1 + 2^-a).
  bf16x8 pf[2][2];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < kBlocks; ++kb) {
    const bool diag = kb == 0 ? kDiag0 : kDiag1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float av = s[kb][r] * k2;
      const float den = 1.0f + __builtin_amdgcn_exp2f(-av);
      float p = __builtin_amdgcn_exp2f(av * __builtin_amdgcn_rcpf(den) - m2);
      if (diag) p = (8 * (r >> 2) + 4 * hf + (r & 3)) < lq ? p : 0.0f;
      pf[kb][r >> 3][r & 7] = (__bf16)p;
    }
    // Row-sum share from the bf16 weights; two independent partial sums.
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      acc0 = __builtin_amdgcn_fdot2_f32_bf16(pf[kb][ks].s01, ones, acc0, false);
      acc1 = __builtin_amdgcn_fdot2_f32_bf16(pf[kb][ks].s23, ones, acc1, false);
      acc0 = __builtin_amdgcn_fdot2_f32_bf16(pf[kb][ks].s45, ones, acc0, false);
      acc1 = __builtin_amdgcn_fdot2_f32_bf16(pf[kb][ks].s67, ones, acc1, false);
    }
    lsum += acc0 + acc1;
  }

  // Transport: O^T[d][q] += V^T[d][key] P^T[key][q]; the key order inside an
  // MFMA k-step matches the register order of the evidence tile.
#pragma unroll
  for (int kb = 0; kb < kBlocks; ++kb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const char* p = vl + voff + (kb * 32 + 16 * ks) * C::kPitchV + 64 * db;
        bf16x8 vf;
        vf.lo = lds_tr_read(p);
        vf.hi = lds_tr_read(p + 8 * C::kPitchV);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][ks], o[db], 0, 0, 0);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(FwdArgs a, HeadParams hp) {
  using C = Cfg<D>;
  constexpr int kDs = D / 16;
  constexpr int kDb = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kBufBytes];

  const int T = a.T;
  const int nq = (T + kBM - 1) / kBM;
  int qt, bh;
  tile_of_block(blockIdx.x, nq, a.B * a.H, qt, bh);
  const int h = bh % a.H;
  const size_t head = (size_t)bh * (size_t)T * D;
  const long long head_bytes = (long long)T * D * 2;
  const __bf16* P1 = static_cast<const __bf16*>(a.P1) + head;
  const __bf16* P2 = static_cast<const __bf16*>(a.P2) + head;
  const __bf16* V = static_cast<const __bf16*>(a.V) + head;
  __bf16* Y = static_cast<__bf16*>(a.Y) + head;
  const auto rP1 = rsrc(P1, head_bytes);
  const auto rP2 = rsrc(P2, head_bytes);
  const auto rV = rsrc(V, head_bytes);
  const auto rY = rsrc(Y, head_bytes);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;                      // query (column) within the wave
  const int hf = lane >> 5;                      // lane half
  const int q0 = qt * kBM;
  const int qrow = q0 + wave * 32 + lq;          // may be >= T: loads give 0, stores drop

  // P1 rows as the evidence MFMA's B operand: lane holds p1[qrow][16 ds + 8 hf + 0..7].
  const int qoff = qrow * (D * 2) + hf * 16;
  bf16x8 qf[kDs];
#pragma unroll
  for (int ds = 0; ds < kDs; ++ds)
    qf[ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP1, qoff + ds * 32, 0, 0));

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
  const int tfull = min(2 * qt, ntiles);         // tiles left of every wave's diagonal

  // Staging: pass `it` moves rows it * kRowsPerPass + tid / kChunks, chunk tid % kChunks.
  const int srow = tid / C::kChunks, sch = tid % C::kChunks;
  const int goff = srow * (D * 2) + sch * 16;
  const int kwoff = srow * C::kPitchK + sch * 16;
  const int vwoff = C::kKBytes + srow * C::kPitchV + sch * 16;
  u32x4 kreg[C::kLoads], vreg[C::kLoads];
  auto gload = [&](int t) {
    const long long base = (long long)t * kBN * D * 2;
    const auto rK = rsrc(P2 + (size_t)t * kBN * D, head_bytes - base);
    const auto rVt = rsrc(V + (size_t)t * kBN * D, head_bytes - base);
#pragma unroll
    for (int it = 0; it < C::kLoads; ++it) {
      kreg[it] = __builtin_amdgcn_raw_buffer_load_b128(rK, goff + it * C::kRowsPerPass * D * 2, 0, 0);
      vreg[it] = __builtin_amdgcn_raw_buffer_load_b128(rVt, goff + it * C::kRowsPerPass * D * 2, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    char* b = smem + buf * C::kBufBytes;
#pragma unroll
    for (int it = 0; it < C::kLoads; ++it) {
      *reinterpret_cast<u32x4*>(b + kwoff + it * C::kRowsPerPass * C::kPitchK) = kreg[it];
      *reinterpret_cast<u32x4*>(b + vwoff + it * C::kRowsPerPass * C::kPitchV) = vreg[it];
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  // Lane-constant read offsets: evidence operand rows (lq, chunk hf) and the
  // transposed V read (16-lane group g supplies rows 4 (g / 2) + i / 4 and
  // columns 16 (g % 2) + 4 (i % 4), i = lane % 16).
  const int koff = lq * C::kPitchK + hf * 16;
  const int tg = lane >> 4, ti = lane & 15;
  const int voff = C::kKBytes + (4 * (tg >> 1) + (ti >> 2)) * C::kPitchV + (16 * (tg & 1) + 4 * (ti & 3)) * 2;

  for (int t = 0; t < ntiles; ++t) {
    const char* lb = smem + (t & 1) * C::kBufBytes;
    // Prefetch the next tile unconditionally: past the last tile the
    // descriptor has no records, so the loads return zeros without touching
    // memory, and no branch separates the loads from the compute below.
    gload(t + 1);
    int mode = 0;
    if (t >= tfull) {
      const int d = t - 2 * qt;                  // 0 or 1: the two tiles holding diagonals
      const int w = wave - 2 * d;                // wave's diagonal block relative to the tile
      mode = w < 0 ? 3 : (w == 0 ? 2 : (w == 1 ? 1 : 0));
    }
    if (mode == 0) {
      tile_step<D, 0>(lb, lb, qf, o, m2, lsum, k2, lq, hf, koff, voff);
    } else if (mode == 1) {
      tile_step<D, 1>(lb, lb, qf, o, m2, lsum, k2, lq, hf, koff, voff);
    } else if (mode == 2) {
      tile_step<D, 2>(lb, lb, qf, o, m2, lsum, k2, lq, hf, koff, voff);
    }
    // The other buffer was last read in tile t - 1, before the previous
    // barrier, so it can be overwritten now (with zeros after the last tile).
    lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  lsum = lane_pair_sum(lsum);
  float dself = 0.0f;
#pragma unroll
  for (int ds = 0; ds < kDs; ++ds) {
    const bf16x8 kv = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rP2, qoff + ds * 32, 0, 0));
#pragma unroll
    for (int e = 0; e < 8; ++e) dself = fmaf((float)qf[ds][e], (float)kv[e], dself);
  }
  dself = lane_pair_sum(dself);
  const float S = sigmoid_f32(dself * hp.scale * hp.inv_tau[h]);
  const RowCombine c(S, m2 * kLn2, lsum, hp.lambda * logf((float)(qrow + 1)));
  const int roff = qrow * (D * 2) + hf * 8;
#pragma unroll
  for (int db = 0; db < kDb; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int boff = roff + (32 * db + 8 * g4) * 2;
      const bf16x4 vv = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rV, boff, 0, 0));
      bf16x4 yy;
#pragma unroll
      for (int e = 0; e < 4; ++e) yy[e] = (__bf16)(c.w_self * (float)vv[e] + c.w_hist * o[db][4 * g4 + e]);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, yy), rY, boff, 0, 0);
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

bool fwd_mfma_supported(int d_h, int T) {
  // Buffer descriptors address one head with 31-bit byte offsets, including
  // the rows past T of the last query tile.
  return (d_h == 64 || d_h == 128) && ((long long)T + kBM) * d_h * 2 < 0x7fffffffLL;
}

hipError_t launch_fwd_mfma_bf16(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  switch (a.d_h) {
    case 64: return launch_typed<64>(a, hp, s);
    case 128: return launch_typed<128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

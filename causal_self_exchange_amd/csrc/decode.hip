// Relation Cache decode ("Ask Self, Ask Others: Relation Is All You Need",
// Sec. 5.3, Eq. (18); App. A.5): one new row per (sequence, head) against the
// cached P2 and information rows.
//
// The step is a stream over the cache, so it is split along the history:
//   decode_partial: n_chunks work-groups per (head, sequence); work-group c
//     scans the blocks of GROUPS cached rows c, c + n_chunks, c + 2 n_chunks,
//     ... and leaves a partial state (m, l, z[d_h]) in the workspace. The
//     interleaving keeps the work-groups of one head sweeping the same part of
//     the cache together, which streams from HBM faster than each work-group
//     reading a separate stretch. Each row is read by d_h/VEC lanes with
//     16-byte loads, so a wave reads whole rows; every row group keeps kAhead
//     rows of loads in flight. The scan uses the log2 domain and the lazy
//     non-negative stabiliser of the forward kernel (m starts at 0 and moves
//     only when a score exceeds it by more than 2^8).
//   decode_merge: one wave per (head, sequence) merges the partial states
//     (the scan update of Eq. (12) applied to whole chunks), adds the Self
//     entry of the new token and the count term for position L + 1, and
//     writes y.
// relation_cache_append implements the cache update of App. A.5.3.
#include <atomic>

#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

constexpr int kPartialThreads = 256;
constexpr int kAhead = 4;                       // rows per row group loaded ahead of use
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;

template <typename Tin>
struct Vec16 {
  static constexpr int N = 16 / sizeof(Tin);
  Tin v[N];
};

template <typename Tin>
__device__ __forceinline__ Vec16<Tin> load16(const Tin* p) {
  Vec16<Tin> out;
  *reinterpret_cast<uint4*>(out.v) = *reinterpret_cast<const uint4*>(p);
  return out;
}

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Lanes per cached row: 16-byte loads cover D / VEC lanes, rounded up to a
// power of two for the shuffle reduction (for d_h = 48 and 80 the lanes past
// the row load nothing and hold zeros); GROUPS rows per step of a work-group.
template <typename Tin, int D>
struct DecodeGeom {
  static constexpr int VEC = 16 / (int)sizeof(Tin);
  static constexpr int LIVE = D / VEC;
  static constexpr int LPR = LIVE <= 4 ? 4 : (LIVE <= 8 ? 8 : (LIVE <= 16 ? 16 : 32));
  static constexpr int GROUPS = kPartialThreads / LPR;
  static_assert(D % VEC == 0 && LIVE <= 32, "row layout");
};

template <typename Tin, int D>
__global__ __launch_bounds__(kPartialThreads) void decode_partial_kernel(DecodeArgs a, HeadParams hp) {
  using G = DecodeGeom<Tin, D>;
  constexpr int VEC = G::VEC;
  constexpr int LPR = G::LPR;                       // lanes per cached row
  constexpr int GROUPS = G::GROUPS;                 // rows in flight per step
  __shared__ float s_m[GROUPS];
  __shared__ float s_l[GROUPS];
  __shared__ float s_z[GROUPS][D + 1];

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nc = gridDim.x;                         // work-groups per (b, h) = n_chunks
  const int L = clamp_len(a.len[b], a.L_cap);
  if (chunk * GROUPS >= L) return;                  // no rows here; uniform for the block

  const int tid = threadIdx.x;
  const int g = tid / LPR;
  const int sl = tid % LPR;
  const bool live = sl < G::LIVE;                   // lanes past the row read its start, weighted 0
  const int so = live ? sl * VEC : 0;
  const size_t bh = (size_t)b * a.H + h;
  const Tin* p1 = static_cast<const Tin*>(a.p1) + bh * D + so;
  const Tin* cP2 = static_cast<const Tin*>(a.cP2) + bh * (size_t)a.L_cap * D + so;
  const Tin* cV = static_cast<const Tin*>(a.cV) + bh * (size_t)a.L_cap * D + so;

  float q[VEC], z[VEC];
  {
    const Vec16<Tin> t = load16(p1);
#pragma unroll
    for (int e = 0; e < VEC; ++e) { q[e] = live ? to_f32(t.v[e]) : 0.0f; z[e] = 0.0f; }
  }
  const float k2 = hp.scale * kLog2e;               // raw dot -> log2-domain evidence
  float m2 = 0.0f, l = 0.0f;                        // stabiliser (log2 domain), row sum

  const int step = nc * GROUPS;                     // rows between this work-group's blocks
  for (int j0 = chunk * GROUPS + g; j0 < L; j0 += step * kAhead) {
    Vec16<Tin> kp[kAhead], kv[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      // Rows past the end re-read the last row; their weight is zero below.
      const int j = min(j0 + u * step, L - 1);
      kp[u] = load16(cP2 + (size_t)j * D);
      kv[u] = load16(cV + (size_t)j * D);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) part = fmaf(q[e], to_f32(kp[u].v[e]), part);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
      // SiLU(u) log2 e = a / (1 + 2^-a), a = u log2 e.
      const float av = part * k2;
      const float e2 = av * __builtin_amdgcn_rcpf(1.0f + exp2f(-av));
      const bool valid = j0 + u * step < L;
      if (valid && e2 > m2 + kLazy) {
        const float al = exp2f(m2 - e2);
        l *= al;
#pragma unroll
        for (int e = 0; e < VEC; ++e) z[e] *= al;
        m2 = e2;
      }
      const float p = valid ? exp2f(e2 - m2) : 0.0f;
      l += p;
#pragma unroll
      for (int e = 0; e < VEC; ++e) z[e] = fmaf(p, to_f32(kv[u].v[e]), z[e]);
    }
  }
  const float m = m2 * kLn2;                        // natural-log stabiliser of this group

  if (sl == 0) { s_m[g] = m; s_l[g] = l; }
  if (live) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_z[g][sl * VEC + e] = z[e];
  }
  __syncthreads();

  float* out = a.ws + (bh * a.n_chunks + chunk) * (size_t)(D + 2);
  for (int k = tid; k < D; k += kPartialThreads) {
    float M = kEmptyMax;
    for (int gg = 0; gg < GROUPS; ++gg) M = fmaxf(M, s_m[gg]);
    float zs = 0.0f, ls = 0.0f;
    for (int gg = 0; gg < GROUPS; ++gg) {
      const float w = expf(s_m[gg] - M);
      zs = fmaf(w, s_z[gg][k], zs);
      ls = fmaf(w, s_l[gg], ls);
    }
    out[2 + k] = zs;
    if (k == 0) { out[0] = M; out[1] = ls; }
  }
}

template <typename Tin, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a, HeadParams hp) {
  constexpr int PER = (D + 63) / 64;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const size_t bh = (size_t)b * a.H + h;
  // The new token's states do not depend on the partials: load them first.
  const Tin* p1 = static_cast<const Tin*>(a.p1) + bh * D;
  const Tin* p2 = static_cast<const Tin*>(a.p2) + bh * D;
  const Tin* v = static_cast<const Tin*>(a.v) + bh * D;
  float p1v[PER], p2v[PER], vv[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int k = lane + 64 * t;
    p1v[t] = k < D ? to_f32(p1[k]) : 0.0f;
    p2v[t] = k < D ? to_f32(p2[k]) : 0.0f;
    vv[t] = k < D ? to_f32(v[k]) : 0.0f;
  }
  constexpr int GROUPS = DecodeGeom<Tin, D>::GROUPS;                         // rows per block
  const int L = clamp_len(a.len[b], a.L_cap);
  // Work-groups that found rows (and wrote a state).
  const int nch = min(a.n_chunks, (L + GROUPS - 1) / GROUPS);
  const float* ws = a.ws + bh * a.n_chunks * (size_t)(D + 2);

  // Online merge of the chunk states (the scan update of Eq. (12) applied to
  // whole chunks); unrolled so that several chunks' loads are in flight.
  float M = kEmptyMax, lsum = 0.0f;
  float zsum[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) zsum[t] = 0.0f;
#pragma unroll 4
  for (int c = 0; c < nch; ++c) {
    const float* st = ws + c * (D + 2);
    const float mc = st[0], lc = st[1];
    float zc[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int k = lane + 64 * t;
      zc[t] = k < D ? st[2 + k] : 0.0f;
    }
    const float Mn = fmaxf(M, mc);
    const float wo = expf(M - Mn), wc = expf(mc - Mn);
    lsum = lsum * wo + lc * wc;
#pragma unroll
    for (int t = 0; t < PER; ++t) zsum[t] = zsum[t] * wo + zc[t] * wc;
    M = Mn;
  }

  Tin* y = static_cast<Tin*>(a.y) + bh * D;
  float dself = 0.0f;
#pragma unroll
  for (int t = 0; t < PER; ++t) dself = fmaf(p1v[t], p2v[t], dself);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dself += __shfl_xor(dself, off);
  const float S = sigmoid_f32(dself * hp.scale * hp.inv_tau[h]);
  const RowCombine cmb(S, M, lsum, hp.lambda * logf((float)(L + 1)));
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int k = lane + 64 * t;
    if (k < D) y[k] = from_f32<Tin>(cmb.w_self * vv[t] + cmb.w_hist * zsum[t]);
  }
}

template <typename Tin>
__global__ __launch_bounds__(256) void cache_append_kernel(Tin* cP2, Tin* cV, int32_t* len,
                                                           const Tin* p2, const Tin* v, int H,
                                                           int L_cap, int D) {
  const int b = blockIdx.x;
  const int L = len[b];
  __syncthreads();                       // every thread has read len[b]
  if (L < 0 || L >= L_cap) return;       // uniform for the block
  for (int idx = threadIdx.x; idx < H * D; idx += blockDim.x) {
    const int h = idx / D, k = idx % D;
    const size_t bh = (size_t)b * H + h;
    cP2[(bh * L_cap + L) * D + k] = p2[bh * D + k];
    cV[(bh * L_cap + L) * D + k] = v[bh * D + k];
  }
  __syncthreads();
  if (threadIdx.x == 0) len[b] = L + 1;
}

template <typename Tin, int D>
hipError_t launch_decode_typed(const DecodeArgs& a, const HeadParams& hp, hipStream_t s) {
  dim3 g1(a.n_chunks, a.H, a.B);
  hipLaunchKernelGGL((decode_partial_kernel<Tin, D>), g1, dim3(kPartialThreads), 0, s, a, hp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(a.H, a.B);
  hipLaunchKernelGGL((decode_merge_kernel<Tin, D>), g2, dim3(64), 0, s, a, hp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const HeadParams& hp, bool bf16, hipStream_t s) {
  switch (a.d_h) {
    case 32: return bf16 ? launch_decode_typed<__bf16, 32>(a, hp, s) : launch_decode_typed<float, 32>(a, hp, s);
    case 48: return bf16 ? launch_decode_typed<__bf16, 48>(a, hp, s) : launch_decode_typed<float, 48>(a, hp, s);
    case 64: return bf16 ? launch_decode_typed<__bf16, 64>(a, hp, s) : launch_decode_typed<float, 64>(a, hp, s);
    case 80: return bf16 ? launch_decode_typed<__bf16, 80>(a, hp, s) : launch_decode_typed<float, 80>(a, hp, s);
    case 128: return bf16 ? launch_decode_typed<__bf16, 128>(a, hp, s) : launch_decode_typed<float, 128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

// Partial states of relation_decode_noalloc: a file-scope device array (each
// GPU the library runs on holds its own copy until the process ends). In host
// code its name is a stand-in, not a device address: the address comes from
// hipGetSymbolAddress, looked up once per device with that device current and
// kept per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::atomic<void*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev].store(p, std::memory_order_release);   // concurrent first calls store the same address
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_cache_append(void* cP2, void* cV, int32_t* len, const void* p2, const void* v,
                               int B, int H, int L_cap, int d_h, bool bf16, hipStream_t s) {
  if (bf16) {
    hipLaunchKernelGGL(cache_append_kernel<__bf16>, dim3(B), dim3(256), 0, s,
                       static_cast<__bf16*>(cP2), static_cast<__bf16*>(cV), len,
                       static_cast<const __bf16*>(p2), static_cast<const __bf16*>(v), H, L_cap, d_h);
  } else {
    hipLaunchKernelGGL(cache_append_kernel<float>, dim3(B), dim3(256), 0, s,
                       static_cast<float*>(cP2), static_cast<float*>(cV), len,
                       static_cast<const float*>(p2), static_cast<const float*>(v), H, L_cap, d_h);
  }
  return hipGetLastError();
}

}  // namespace rel

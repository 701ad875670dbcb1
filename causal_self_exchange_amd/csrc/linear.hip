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
// Three kernels: chunk (the bracketed sum and e^{b_last} per chunk), scan
// (the elementwise recurrence over chunks, one thread per state element),
// output (Y per chunk). Arithmetic is fp32 throughout.
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

constexpr int kL = kLinChunk;          // tokens per chunk
constexpr int kThreads = 256;

template <typename Tin>
__device__ __forceinline__ float ld(const Tin* p, size_t i) { return to_f32(p[i]); }

// Row statistics of one chunk: S_t (into s[]), the row norms' reciprocals of
// p1 and p2 (into n1[], n2[]), for rows t < rows; one wave per row at a time.
template <typename Tin, int D>
__device__ __forceinline__ void chunk_rows(const Tin* P1, const Tin* P2, int rows, float inv_scale, float* s,
                                           float* n1, float* n2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < kL; t += kThreads / 64) {
    float d12 = 0.0f, d11 = 0.0f, d22 = 0.0f;
    if (t < rows) {
      for (int r = lane; r < D; r += 64) {
        const float a = ld(P1, (size_t)t * D + r), b = ld(P2, (size_t)t * D + r);
        d12 = fmaf(a, b, d12);
        d11 = fmaf(a, a, d11);
        d22 = fmaf(b, b, d22);
      }
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
      d12 += __shfl_xor(d12, w, 64);
      d11 += __shfl_xor(d11, w, 64);
      d22 += __shfl_xor(d22, w, 64);
    }
    if (lane == 0) {
      s[t] = t < rows ? sigmoid_f32(d12 * inv_scale) : 0.0f;
      // A zero row has no direction: its normalised coordinate is 0.
      n1[t] = d11 > 0.0f ? 1.0f / sqrtf(d11) : 0.0f;
      n2[t] = d22 > 0.0f ? 1.0f / sqrtf(d22) : 0.0f;
    }
  }
}

// Inclusive per-channel prefix of log alpha over the chunk's rows into bt[t][r]
// (rows past the chunk's end repeat the last value). alpha is clamped to
// [1e-30, 1] (NaN to 1e-30): log alpha stays finite, so differences of
// prefixes never form inf - inf, and a retention below 1e-30 already wipes
// the state within one step to fp32 precision.
__device__ __forceinline__ void chunk_decay(const float* A, int rows, int D, float* bt) {
  for (int r = threadIdx.x; r < D; r += kThreads) {
    float acc = 0.0f;
    for (int t = 0; t < kL; ++t) {
      if (t < rows) acc += logf(fminf(fmaxf(A[(size_t)t * D + r], 1e-30f), 1.0f));
      bt[t * D + r] = acc;
    }
  }
}

// Phase 1: per (b*H + h, chunk): dC = sum_j S_j (k_j o e^{b_last - b_j}) I_j^T
// and g = e^{b_last}, into the state slot of the chunk.
template <typename Tin, int D>
__global__ __launch_bounds__(kThreads) void lin_chunk_kernel(LinArgs a, HeadParams hp) {
  __shared__ float kt[kL][D];     // S_j k_j e^{b_last - b_j}
  __shared__ float it[kL][D];     // I_j
  __shared__ float bt[kL * D];
  __shared__ float s[kL], n1[kL], n2[kL];
  const int nc = (a.T + kL - 1) / kL;
  const int c = blockIdx.x % nc;
  const int bh = blockIdx.x / nc;
  const int h = bh % a.H;
  const int t0 = c * kL;
  const int rows = min(kL, a.T - t0);
  const size_t base = ((size_t)bh * a.T + t0) * D;
  const Tin* P1 = static_cast<const Tin*>(a.P1) + base;
  const Tin* P2 = static_cast<const Tin*>(a.P2) + base;
  const Tin* I = static_cast<const Tin*>(a.I) + base;
  const float* A = a.alpha + base;

  chunk_rows<Tin, D>(P1, P2, rows, hp.scale * hp.inv_tau[h], s, n1, n2);
  chunk_decay(A, rows, D, bt);
  __syncthreads();
  for (int e = threadIdx.x; e < kL * D; e += kThreads) {
    const int t = e / D, r = e % D;
    const bool v = t < rows;
    const float blast = bt[(kL - 1) * D + r];
    kt[t][r] = v ? s[t] * ld(P2, (size_t)t * D + r) * n2[t] * __expf(blast - bt[t * D + r]) : 0.0f;
    it[t][r] = v ? ld(I, (size_t)t * D + r) : 0.0f;
  }
  __syncthreads();
  // dC[r][col]: each thread a block of rows r and 4 consecutive columns.
  float* dC = a.state + ((size_t)bh * nc + c) * (size_t)D * D;
  constexpr int kCols = 4;
  for (int o = threadIdx.x; o < D * D / kCols; o += kThreads) {
    const int r = o / (D / kCols), c4 = (o % (D / kCols)) * kCols;
    float acc[kCols] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < kL; ++j) {
      const float kv = kt[j][r];
#pragma unroll
      for (int u = 0; u < kCols; ++u) acc[u] = fmaf(kv, it[j][c4 + u], acc[u]);
    }
    *reinterpret_cast<float4*>(dC + (size_t)r * D + c4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
  if (threadIdx.x < D) a.decay[((size_t)bh * nc + c) * D + threadIdx.x] = __expf(bt[(kL - 1) * D + threadIdx.x]);
}

// Phase 2: per state element (b*H + h, r, col): Cin_0 = 0,
// Cin_{c+1} = e^{b_last,c}[r] Cin_c + dC_c; each chunk slot is overwritten
// with its entering state, and the final state goes to a.final (if given).
template <int D>
__global__ __launch_bounds__(kThreads) void lin_scan_kernel(LinArgs a) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)a.B * a.H * D * D) return;
  const int e = (int)(idx % (D * D));
  const long long bh = idx / (D * D);
  const int r = e / D;
  const int nc = (a.T + kL - 1) / kL;
  float* st = a.state + (size_t)bh * nc * D * D + e;
  const float* g = a.decay + (size_t)bh * nc * D + r;
  float C = 0.0f;
  for (int c = 0; c < nc; ++c) {
    const float dc = st[(size_t)c * D * D];
    st[(size_t)c * D * D] = C;
    C = fmaf(g[(size_t)c * D], C, dc);
  }
  if (a.final) a.final[(size_t)bh * D * D + e] = C;
}

// Phase 3: per (b*H + h, chunk): Y = I + inter + intra.
template <typename Tin, int D>
__global__ __launch_bounds__(kThreads) void lin_out_kernel(LinArgs a, HeadParams hp) {
  __shared__ float q[kL][D];      // q_t, later q_t o e^{b_t}
  __shared__ float k[kL][D];      // S_j k_j
  __shared__ float bt[kL * D];    // b_t (later reused to stage rows of Cin)
  __shared__ float it[kL][D];     // I_j
  __shared__ float at[kL][kL + 1];// intra coefficients S_t S_j (q_t . k_j decayed)
  __shared__ float s[kL], n1[kL], n2[kL];
  const int nc = (a.T + kL - 1) / kL;
  const int c = blockIdx.x % nc;
  const int bh = blockIdx.x / nc;
  const int h = bh % a.H;
  const int t0 = c * kL;
  const int rows = min(kL, a.T - t0);
  const size_t base = ((size_t)bh * a.T + t0) * D;
  const Tin* P1 = static_cast<const Tin*>(a.P1) + base;
  const Tin* P2 = static_cast<const Tin*>(a.P2) + base;
  const Tin* I = static_cast<const Tin*>(a.I) + base;
  const float* A = a.alpha + base;
  Tin* Y = static_cast<Tin*>(a.Y) + base;

  chunk_rows<Tin, D>(P1, P2, rows, hp.scale * hp.inv_tau[h], s, n1, n2);
  chunk_decay(A, rows, D, bt);
  __syncthreads();
  for (int e = threadIdx.x; e < kL * D; e += kThreads) {
    const int t = e / D, r = e % D;
    const bool v = t < rows;
    q[t][r] = v ? ld(P1, (size_t)t * D + r) * n1[t] : 0.0f;
    k[t][r] = v ? s[t] * ld(P2, (size_t)t * D + r) * n2[t] : 0.0f;
    it[t][r] = v ? ld(I, (size_t)t * D + r) : 0.0f;
  }
  __syncthreads();
  // Intra-chunk coefficients for j < t (0 elsewhere).
  for (int e = threadIdx.x; e < kL * kL; e += kThreads) {
    const int t = e / kL, j = e % kL;
    float acc = 0.0f;
    if (j < t && t < rows) {
      for (int r = 0; r < D; ++r) acc = fmaf(q[t][r] * k[j][r], __expf(bt[t * D + r] - bt[j * D + r]), acc);
      acc *= s[t];
    }
    at[t][j] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kL * D; e += kThreads) {
    const int t = e / D, r = e % D;
    q[t][r] *= __expf(bt[t * D + r]);
  }
  // Outputs: thread handles 4 consecutive columns of 2 rows per pass.
  constexpr int kCols = 4;
  constexpr int kRowsPer = 2;
  const float* cin = a.state + ((size_t)bh * nc + c) * (size_t)D * D;
  float* stage = bt;              // rows r0 .. r0 + kStage - 1 of Cin
  constexpr int kStage = D < kL ? D : kL;   // rows of Cin staged at a time (D % kStage == 0)
  static_assert(kStage * D <= kL * D && D % kStage == 0, "staging fits");
  for (int base_o = 0; base_o < kL * D / (kCols * kRowsPer); base_o += kThreads) {
    const int o = base_o + threadIdx.x;
    const bool act = o < kL * D / (kCols * kRowsPer);
    const int tp = act ? o / (D / kCols) : 0;            // row pair
    const int c4 = act ? (o % (D / kCols)) * kCols : 0;
    float acc[kRowsPer][kCols];
#pragma unroll
    for (int x = 0; x < kRowsPer; ++x)
#pragma unroll
      for (int u = 0; u < kCols; ++u) acc[x][u] = 0.0f;
    // Intra: sum_j at[t][j] I_j.
    for (int j = 0; j < kL; ++j) {
#pragma unroll
      for (int x = 0; x < kRowsPer; ++x) {
        const float w = at[kRowsPer * tp + x][j];
#pragma unroll
        for (int u = 0; u < kCols; ++u) acc[x][u] = fmaf(w, it[j][c4 + u], acc[x][u]);
      }
    }
    // Inter: S_t sum_r (q_t o e^{b_t})_r Cin[r][col], Cin staged kL rows at a time.
    float inter[kRowsPer][kCols];
#pragma unroll
    for (int x = 0; x < kRowsPer; ++x)
#pragma unroll
      for (int u = 0; u < kCols; ++u) inter[x][u] = 0.0f;
    for (int r0 = 0; r0 < D; r0 += kStage) {
      __syncthreads();
      for (int e = threadIdx.x; e < kStage * D; e += kThreads) stage[e] = cin[(size_t)r0 * D + e];
      __syncthreads();
      if (act) {
        for (int rr = 0; rr < kStage; ++rr) {
#pragma unroll
          for (int x = 0; x < kRowsPer; ++x) {
            const float w = q[kRowsPer * tp + x][r0 + rr];
#pragma unroll
            for (int u = 0; u < kCols; ++u) inter[x][u] = fmaf(w, stage[rr * D + c4 + u], inter[x][u]);
          }
        }
      }
    }
    if (act) {
#pragma unroll
      for (int x = 0; x < kRowsPer; ++x) {
        const int t = kRowsPer * tp + x;
        if (t < rows) {
#pragma unroll
          for (int u = 0; u < kCols; ++u)
            Y[(size_t)t * D + c4 + u] = from_f32<Tin>(it[t][c4 + u] + fmaf(s[t], inter[x][u], acc[x][u]));
        }
      }
    }
  }
}

template <typename Tin, int D>
hipError_t launch_typed(const LinArgs& a, const HeadParams& hp, hipStream_t s) {
  const int nc = (a.T + kL - 1) / kL;
  const long long wg = (long long)a.B * a.H * nc;
  const long long scan_threads = (long long)a.B * a.H * D * D;
  if (wg > 0x7fffffffLL || (scan_threads + kThreads - 1) / kThreads > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((lin_chunk_kernel<Tin, D>), dim3((unsigned)wg), dim3(kThreads), 0, s, a, hp);
  hipLaunchKernelGGL((lin_scan_kernel<D>), dim3((unsigned)((scan_threads + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((lin_out_kernel<Tin, D>), dim3((unsigned)wg), dim3(kThreads), 0, s, a, hp);
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

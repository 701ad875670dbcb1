// Backward of the causal Self-Exchange Relation: the row-statistics prep, the
// fixed-order reduction of the scalar gradients, and a row-per-lane backward
// for fp32 and for head sizes without an MFMA kernel.
//
// Gradients of L = sum_i dY_i . Y_i through the operator of "Ask Self, Ask
// Others: Relation Is All You Need", Eq. (1)-(3), recomputing U per key from
// the stored per-row log normaliser (the FlashRelation backward of App. A.3
// recomputes the scan's evidence the same way). With F = softmax(R) row-wise:
//   D_i   = dY_i . Y_i  (= sum_j F_ij dF_ij)
//   dF_ij = dY_i . V_j,        dR_ij = F_ij (dF_ij - D_i)
//   dU_ij = dR_ij SiLU'(U_ij)  for j < i,  SiLU'(x) = s(x) (1 + x (1 - s(x)))
//   dU_ii = dR_ii S_i (1 - S_i) / tau,     S_i = sigmoid(U_ii / tau)
//   dP1_i = sum_j dU_ij p2_j / sqrt(d_h),  dP2_j = sum_i dU_ij p1_i / sqrt(d_h)
//   dV_j  = sum_i F_ij dY_i
//   dtau  = sum_i dR_ii S_i (1 - S_i) (-U_ii / tau^2)
//   dlambda = -sum_i log i sum_{j<i} dR_ij = sum_i log i dR_ii
// (the last step because every row of dR sums to zero: sum_j F_ij = 1).
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr int kPrepThreads = 256;

__device__ __forceinline__ int64_t stat_index(int64_t bh, int nt, int r, int k) {
  return ((bh * nt + r / kStatRows) * 4 + k) * kStatRows + (r % kStatRows);
}

// 8 consecutive elements of a row as fp32.
template <typename Tin>
__device__ __forceinline__ void load8(const Tin* p, float (&x)[8]) {
  if constexpr (sizeof(Tin) == 2) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Prep: one work-group per (256-row chunk, b*H + h); D/8 lanes per row, each
// lane 8 consecutive columns. Writes the row statistics (rows past T of the
// last 64-row tile get the padding values) and one (dtau, dlambda) partial.
template <typename Tin, int D>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(BwdArgs a, HeadParams hp) {
  // Lanes per row: D / 8 loading lanes, rounded up to a power of two for the
  // shuffle reduction (the extra lanes contribute 0).
  constexpr int kUsed = D / 8;
  constexpr int kLpr = kUsed <= 4 ? 4 : (kUsed <= 8 ? 8 : 16);
  constexpr int kRowsPerPass = kPrepThreads / kLpr;
  static_assert(kUsed <= kLpr && kPrepRows % kRowsPerPass == 0, "prep lane layout");
  __shared__ float red[2][kPrepThreads / 64];

  const int T = a.T;
  const int nch = (T + kPrepRows - 1) / kPrepRows;
  const int chunk = (int)(blockIdx.x % nch);
  const int bh = (int)(blockIdx.x / nch);
  const int h = bh % a.H;
  const int nt = (T + kStatRows - 1) / kStatRows;
  const int tid = threadIdx.x;
  const int sub = tid % kLpr;
  const size_t head = (size_t)bh * (size_t)T * D;
  const Tin* P1 = static_cast<const Tin*>(a.P1) + head;
  const Tin* P2 = static_cast<const Tin*>(a.P2) + head;
  const Tin* V = static_cast<const Tin*>(a.V) + head;
  const Tin* Y = static_cast<const Tin*>(a.Y) + head;
  const Tin* dY = static_cast<const Tin*>(a.dY) + head;
  const float inv_tau = hp.inv_tau[h];

  float part_tau = 0.0f, part_lam = 0.0f;
  for (int pass = 0; pass < kPrepRows / kRowsPerPass; ++pass) {
    const int r = chunk * kPrepRows + pass * kRowsPerPass + tid / kLpr;
    float dyy = 0.0f, p12 = 0.0f, dyv = 0.0f;
    if (r < T && sub < kUsed) {
      float x[8], y[8];
      const size_t off = (size_t)r * D + 8 * sub;
      load8(dY + off, x);
      load8(Y + off, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) dyy = fmaf(x[e], y[e], dyy);
      load8(V + off, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) dyv = fmaf(x[e], y[e], dyv);
      load8(P1 + off, x);
      load8(P2 + off, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) p12 = fmaf(x[e], y[e], p12);
    }
#pragma unroll
    for (int w = 1; w < kLpr; w <<= 1) {
      dyy += __shfl_xor(dyy, w, kLpr);
      dyv += __shfl_xor(dyv, w, kLpr);
      p12 += __shfl_xor(p12, w, kLpr);
    }
    if (sub == 0 && r < nt * kStatRows) {
      float st[4];
      if (r < T) {
        const float lse = a.lse[(size_t)bh * T + r];
        const float logi = logf((float)(r + 1));
        const float u = p12 * hp.scale;                 // U_ii
        const float S = sigmoid_f32(u * inv_tau);
        const float Fs = expf(S - lse);                 // F_ii
        const float dR = Fs * (dyv - dyy);              // dR_ii
        const float sp = S * (1.0f - S);
        st[0] = (lse + hp.lambda * logi) * kLog2eF;
        st[1] = -dyy;
        st[2] = Fs;
        st[3] = dR * sp * inv_tau * hp.scale;
        part_tau += dR * sp * (-u * inv_tau * inv_tau);
        part_lam += logi * dR;
      } else {
        st[0] = INFINITY;
        st[1] = st[2] = st[3] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) a.stats[stat_index(bh, nt, r, k)] = st[k];
    }
  }
  // Fixed-order block reduction of the partials.
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) {
    part_tau += __shfl_xor(part_tau, w, 64);
    part_lam += __shfl_xor(part_lam, w, 64);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = part_tau;
    red[1][tid >> 6] = part_lam;
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f, l = 0.0f;
    for (int w = 0; w < kPrepThreads / 64; ++w) {
      t += red[0][w];
      l += red[1][w];
    }
    a.part[((size_t)bh * nch + chunk) * 2 + 0] = t;
    a.part[((size_t)bh * nch + chunk) * 2 + 1] = l;
  }
}

// dtau[h] = sum over b and chunks of the partials (in that order, fp64);
// dlambda = sum over h of the per-head lambda sums (in order of h).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  __shared__ double lam[256];
  const int nch = (a.T + kPrepRows - 1) / kPrepRows;
  const int h = threadIdx.x;
  double lh = 0.0;
  if (h < a.H) {
    double t = 0.0;
    for (int b = 0; b < a.B; ++b) {
      const float* p = a.part + ((size_t)b * a.H + h) * nch * 2;
      for (int c = 0; c < nch; ++c) {
        t += (double)p[2 * c];
        lh += (double)p[2 * c + 1];
      }
    }
    a.dtau[h] = (float)t;
  }
  lam[h] = lh;
  __syncthreads();
  if (h == 0) {
    double l = 0.0;
    for (int k = 0; k < a.H; ++k) l += lam[k];
    a.dlambda[0] = (float)l;
  }
}

// ---------------------------------------------------------------------------
// Row-per-lane backward (fp32 FMA).
// ---------------------------------------------------------------------------

constexpr int kRows = 64;   // rows per work-group (one wave)
constexpr int kKeys = 32;   // rows per LDS tile

// Query gradient: lane = query row i, scanning keys j < i.
template <typename Tin, int D>
__global__ __launch_bounds__(kRows) void bwd_scan_dq_kernel(BwdArgs a, HeadParams hp) {
  __shared__ float sP2[kKeys][D];
  __shared__ float sV[kKeys][D];
  const int lane = threadIdx.x;
  const int bh = blockIdx.z * a.H + blockIdx.y;
  const int T = a.T;
  const int nt = (T + kStatRows - 1) / kStatRows;
  const int row0 = blockIdx.x * kRows;
  const int r = row0 + lane;
  const bool valid = r < T;
  const size_t head = (size_t)bh * (size_t)T * D;
  const Tin* P1 = static_cast<const Tin*>(a.P1) + head;
  const Tin* P2 = static_cast<const Tin*>(a.P2) + head;
  const Tin* V = static_cast<const Tin*>(a.V) + head;
  const Tin* dY = static_cast<const Tin*>(a.dY) + head;
  Tin* dP1 = static_cast<Tin*>(a.dP1) + head;

  float q[D], dy[D], acc[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    q[k] = valid ? to_f32(P1[(size_t)r * D + k]) : 0.0f;
    dy[k] = valid ? to_f32(dY[(size_t)r * D + k]) : 0.0f;
    acc[k] = 0.0f;
  }
  const float L2 = valid ? a.stats[stat_index(bh, nt, r, 0)] : 0.0f;
  const float negD = valid ? a.stats[stat_index(bh, nt, r, 1)] : 0.0f;

  const int last = min(T - 1, row0 + kRows - 1);
  for (int j0 = 0; j0 < last; j0 += kKeys) {
    for (int e = lane; e < kKeys * D; e += kRows) {
      const int jj = e / D, k = e % D;
      const int j = j0 + jj;
      sP2[jj][k] = j < T ? to_f32(P2[(size_t)j * D + k]) : 0.0f;
      sV[jj][k] = j < T ? to_f32(V[(size_t)j * D + k]) : 0.0f;
    }
    __syncthreads();
    for (int jj = 0; jj < kKeys; ++jj) {
      if (valid && j0 + jj < r) {
        float s = 0.0f, g = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) {
          s = fmaf(q[k], sP2[jj][k], s);
          g = fmaf(dy[k], sV[jj][k], g);
        }
        const float u = s * hp.scale;
        const float sg = sigmoid_f32(u);
        const float F = exp2f(u * sg * kLog2eF - L2);
        const float w = F * (g + negD) * (sg * (1.0f + u * (1.0f - sg)));
#pragma unroll
        for (int k = 0; k < D; ++k) acc[k] = fmaf(w, sP2[jj][k], acc[k]);
      }
    }
    __syncthreads();
  }
  if (!valid) return;
  const float us = a.stats[stat_index(bh, nt, r, 3)];
#pragma unroll
  for (int k = 0; k < D; ++k)
    dP1[(size_t)r * D + k] = from_f32<Tin>(fmaf(acc[k], hp.scale, us * to_f32(P2[(size_t)r * D + k])));
}

// Key gradients: lane = key row j, scanning queries i > j. kDV: dV_j (needs
// only F); otherwise dP2_j (needs dR as well).
template <typename Tin, int D, bool kDV>
__global__ __launch_bounds__(kRows) void bwd_scan_dkv_kernel(BwdArgs a, HeadParams hp) {
  __shared__ float sP1[kKeys][D];
  __shared__ float sdY[kKeys][D];
  __shared__ float sL2[kKeys], snD[kKeys];
  const int lane = threadIdx.x;
  const int bh = blockIdx.z * a.H + blockIdx.y;
  const int T = a.T;
  const int nt = (T + kStatRows - 1) / kStatRows;
  const int key0 = blockIdx.x * kRows;
  const int j = key0 + lane;
  const bool valid = j < T;
  const size_t head = (size_t)bh * (size_t)T * D;
  const Tin* P1 = static_cast<const Tin*>(a.P1) + head;
  const Tin* P2 = static_cast<const Tin*>(a.P2) + head;
  const Tin* V = static_cast<const Tin*>(a.V) + head;
  const Tin* dY = static_cast<const Tin*>(a.dY) + head;
  Tin* out = static_cast<Tin*>(kDV ? a.dV : a.dP2) + head;

  float kr[D], vr[kDV ? 1 : D], acc[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    kr[k] = valid ? to_f32(P2[(size_t)j * D + k]) : 0.0f;
    if constexpr (!kDV) vr[k] = valid ? to_f32(V[(size_t)j * D + k]) : 0.0f;
    acc[k] = 0.0f;
  }
  // Only queries i > key0 see a key of this block.
  for (int i0 = key0; i0 < T; i0 += kKeys) {
    for (int e = lane; e < kKeys * D; e += kRows) {
      const int ii = e / D, k = e % D;
      const int i = i0 + ii;
      sP1[ii][k] = i < T ? to_f32(P1[(size_t)i * D + k]) : 0.0f;
      sdY[ii][k] = i < T ? to_f32(dY[(size_t)i * D + k]) : 0.0f;
    }
    if (lane < kKeys) {
      const int i = i0 + lane;
      sL2[lane] = i < T ? a.stats[stat_index(bh, nt, i, 0)] : INFINITY;
      snD[lane] = i < T ? a.stats[stat_index(bh, nt, i, 1)] : 0.0f;
    }
    __syncthreads();
    for (int ii = 0; ii < kKeys; ++ii) {
      if (valid && i0 + ii > j && i0 + ii < T) {
        float s = 0.0f, g = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) s = fmaf(kr[k], sP1[ii][k], s);
        if constexpr (!kDV) {
#pragma unroll
          for (int k = 0; k < D; ++k) g = fmaf(vr[k], sdY[ii][k], g);
        }
        const float u = s * hp.scale;
        const float sg = sigmoid_f32(u);
        const float F = exp2f(u * sg * kLog2eF - sL2[ii]);
        if constexpr (kDV) {
#pragma unroll
          for (int k = 0; k < D; ++k) acc[k] = fmaf(F, sdY[ii][k], acc[k]);
        } else {
          const float w = F * (g + snD[ii]) * (sg * (1.0f + u * (1.0f - sg)));
#pragma unroll
          for (int k = 0; k < D; ++k) acc[k] = fmaf(w, sP1[ii][k], acc[k]);
        }
      }
    }
    __syncthreads();
  }
  if (!valid) return;
  if constexpr (kDV) {
    const float fs = a.stats[stat_index(bh, nt, j, 2)];
#pragma unroll
    for (int k = 0; k < D; ++k) out[(size_t)j * D + k] = from_f32<Tin>(fmaf(fs, to_f32(dY[(size_t)j * D + k]), acc[k]));
  } else {
    const float us = a.stats[stat_index(bh, nt, j, 3)];
#pragma unroll
    for (int k = 0; k < D; ++k)
      out[(size_t)j * D + k] = from_f32<Tin>(fmaf(acc[k], hp.scale, us * to_f32(P1[(size_t)j * D + k])));
  }
}

template <typename Tin, int D>
hipError_t launch_prep_typed(const BwdArgs& a, const HeadParams& hp, hipStream_t s) {
  dim3 grid((unsigned)(((a.T + kPrepRows - 1) / kPrepRows) * (long long)a.B * a.H));
  hipLaunchKernelGGL((bwd_prep_kernel<Tin, D>), grid, dim3(kPrepThreads), 0, s, a, hp);
  return hipGetLastError();
}

template <typename Tin, int D>
hipError_t launch_scan_typed(const BwdArgs& a, const HeadParams& hp, hipStream_t s) {
  dim3 grid((a.T + kRows - 1) / kRows, a.H, a.B);
  hipLaunchKernelGGL((bwd_scan_dq_kernel<Tin, D>), grid, dim3(kRows), 0, s, a, hp);
  hipLaunchKernelGGL((bwd_scan_dkv_kernel<Tin, D, true>), grid, dim3(kRows), 0, s, a, hp);
  hipLaunchKernelGGL((bwd_scan_dkv_kernel<Tin, D, false>), grid, dim3(kRows), 0, s, a, hp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s) {
  switch (a.d_h) {
    case 32: return bf16 ? launch_prep_typed<__bf16, 32>(a, hp, s) : launch_prep_typed<float, 32>(a, hp, s);
    case 48: return bf16 ? launch_prep_typed<__bf16, 48>(a, hp, s) : launch_prep_typed<float, 48>(a, hp, s);
    case 64: return bf16 ? launch_prep_typed<__bf16, 64>(a, hp, s) : launch_prep_typed<float, 64>(a, hp, s);
    case 80: return bf16 ? launch_prep_typed<__bf16, 80>(a, hp, s) : launch_prep_typed<float, 80>(a, hp, s);
    case 128: return bf16 ? launch_prep_typed<__bf16, 128>(a, hp, s) : launch_prep_typed<float, 128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_scan(const BwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s) {
  switch (a.d_h) {
    case 32: return bf16 ? launch_scan_typed<__bf16, 32>(a, hp, s) : launch_scan_typed<float, 32>(a, hp, s);
    case 48: return bf16 ? launch_scan_typed<__bf16, 48>(a, hp, s) : launch_scan_typed<float, 48>(a, hp, s);
    case 64: return bf16 ? launch_scan_typed<__bf16, 64>(a, hp, s) : launch_scan_typed<float, 64>(a, hp, s);
    case 80: return bf16 ? launch_scan_typed<__bf16, 80>(a, hp, s) : launch_scan_typed<float, 80>(a, hp, s);
    case 128: return bf16 ? launch_scan_typed<__bf16, 128>(a, hp, s) : launch_scan_typed<float, 128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rel

// Row-per-lane FlashRelation forward: one lane owns one query row and scans
// its Exchange history key by key with an exact running maximum ("Ask Self,
// Ask Others: Relation Is All You Need", Sec. 5.1, Eq. (12)-(14); App. A.3).
//
// This is the fp32 path (fp32 FMA for both contractions) and the fallback for
// head sizes without an MFMA kernel. Key tiles are staged through LDS as
// fp32 and read by every lane of the wave at the same address (broadcast).
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

constexpr int kRows = 64;   // query rows per work-group (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

template <typename Tin, int D>
__global__ __launch_bounds__(kRows) void fwd_scan_kernel(FwdArgs a, HeadParams hp) {
  __shared__ float sP2[kKeys][D];
  __shared__ float sV[kKeys][D];

  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int row0 = blockIdx.x * kRows;
  const int r = row0 + lane;
  const bool valid = r < a.T;
  const size_t head = ((size_t)b * a.H + h) * (size_t)a.T * D;
  const Tin* P1 = static_cast<const Tin*>(a.P1) + head;
  const Tin* P2 = static_cast<const Tin*>(a.P2) + head;
  const Tin* V = static_cast<const Tin*>(a.V) + head;
  Tin* Y = static_cast<Tin*>(a.Y) + head;

  float q[D];
  float z[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    q[k] = valid ? to_f32(P1[(size_t)r * D + k]) : 0.0f;
    z[k] = 0.0f;
  }
  float m = kEmptyMax;
  float l = 0.0f;

  // Keys 0 .. last-1 are history for some row of this block.
  const int last = min(a.T - 1, row0 + kRows - 1);
  for (int j0 = 0; j0 < last; j0 += kKeys) {
    for (int e = lane; e < kKeys * D; e += kRows) {
      const int jj = e / D, k = e % D;
      const int j = j0 + jj;
      sP2[jj][k] = j < a.T ? to_f32(P2[(size_t)j * D + k]) : 0.0f;
      sV[jj][k] = j < a.T ? to_f32(V[(size_t)j * D + k]) : 0.0f;
    }
    __syncthreads();
    for (int jj = 0; jj < kKeys; ++jj) {
      const int j = j0 + jj;
      if (valid && j < r) {
        float dot = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) dot = fmaf(q[k], sP2[jj][k], dot);
        const float E = silu_f32(dot * hp.scale);
        if (E > m) {                       // new running maximum: rescale
          const float s = expf(m - E);
          l *= s;
#pragma unroll
          for (int k = 0; k < D; ++k) z[k] *= s;
          m = E;
        }
        const float p = expf(E - m);
        l += p;
#pragma unroll
        for (int k = 0; k < D; ++k) z[k] = fmaf(p, sV[jj][k], z[k]);
      }
    }
    __syncthreads();
  }

  if (!valid) return;
  // Self entry from the row's own evidence; V_i for the Self share.
  float dself = 0.0f;
#pragma unroll
  for (int k = 0; k < D; ++k) dself = fmaf(q[k], to_f32(P2[(size_t)r * D + k]), dself);
  const float S = sigmoid_f32(dself * hp.scale * hp.inv_tau[h]);
  const RowCombine c(S, m, l, hp.lambda * logf((float)(r + 1)));
  if (a.lse) a.lse[((size_t)b * a.H + h) * (size_t)a.T + r] = c.lse;
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const float vi = to_f32(V[(size_t)r * D + k]);
    Y[(size_t)r * D + k] = from_f32<Tin>(c.w_self * vi + c.w_hist * z[k]);
  }
}

template <typename Tin, int D>
hipError_t launch_typed(const FwdArgs& a, const HeadParams& hp, hipStream_t s) {
  dim3 grid((a.T + kRows - 1) / kRows, a.H, a.B);
  hipLaunchKernelGGL((fwd_scan_kernel<Tin, D>), grid, dim3(kRows), 0, s, a, hp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_scan(const FwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s) {
  switch (a.d_h) {
    case 32: return bf16 ? launch_typed<__bf16, 32>(a, hp, s) : launch_typed<float, 32>(a, hp, s);
    case 48: return bf16 ? launch_typed<__bf16, 48>(a, hp, s) : launch_typed<float, 48>(a, hp, s);
    case 64: return bf16 ? launch_typed<__bf16, 64>(a, hp, s) : launch_typed<float, 64>(a, hp, s);
    case 80: return bf16 ? launch_typed<__bf16, 80>(a, hp, s) : launch_typed<float, 80>(a, hp, s);
    case 128: return bf16 ? launch_typed<__bf16, 128>(a, hp, s) : launch_typed<float, 128>(a, hp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

// Device-side helpers shared by the HIP kernel files of librelation.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rel {

// Finite stand-in for -inf as the empty-history running maximum: exp of
// (sentinel - anything finite) is exactly 0, and it survives any fast-math
// assumption that infinities do not occur.
constexpr float kEmptyMax = -1.0e30f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (gfx950 lowers this to v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// sigmoid(x) = 1 / (1 + e^-x); for x -> -inf e^-x overflows to +inf and the
// quotient is 0, for x -> +inf it is 1, so no branch is needed.
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }
// SiLU(x) = x * sigmoid(x) = x / (1 + e^-x).
__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// Final Self/Exchange combination of one row (paper Eq. (13)-(14)), written
// so that the empty history (m = kEmptyMax, l = 0, z = 0) needs no branch:
//   m' = m - lambda log i,  M = max(m', S),
//   a = e^{S - M},  c = e^{m' - M},
//   Y = (a / (a + c l)) V_i + (c / (a + c l)) z.
// On the first row c = 0, the Self weight is a / a = 1 exactly and Y = V_i.
struct RowCombine {
  float w_self, w_hist;
  float lse;   // log of the row's full normaliser e^S + e^{m - count} l
  __device__ __forceinline__ RowCombine(float S, float m, float l, float count) {
    const float mp = m - count;
    const float M = fmaxf(mp, S);
    const float a = expf(S - M);
    const float c = expf(mp - M);
    const float den = a + c * l;
    w_self = a / den;
    w_hist = c / den;
    lse = M + logf(den);
  }
};

// sin and cos of an angle held in fp64: reduced by pi/2 in fp64 (the
// remainder r, |r| <= pi/4, is exact to far below fp32 resolution for the
// angles a position count produces), then the single-precision minimax
// polynomials for sin and cos on [-pi/4, pi/4] published with S. Moshier's
// Cephes library (sinf / cosf), and the quadrant's swap and signs. Accurate
// to a few fp32 ulps, with none of a general sincosf's large-argument path.
__device__ __forceinline__ void sincos_of(double ang, float* s, float* c) {
  const double k = rint(ang * 0.63661977236758134);           // 2 / pi
  const float r = (float)fma(-k, 1.5707963267948966, ang);     // ang - k pi / 2
  const int q = (int)(long long)k & 3;                          // quadrant (two's complement mod 4)
  const float z = r * r;
  const float sr = fmaf(r * z, fmaf(z, fmaf(z, -1.9515295891e-4f, 8.3321608736e-3f), -1.6666654611e-1f), r);
  const float cr = fmaf(z * z, fmaf(z, fmaf(z, 2.443315711809948e-5f, -1.388731625493765e-3f), 4.166664568298827e-2f),
                        fmaf(-0.5f, z, 1.0f));
  const float sv = (q & 1) ? cr : sr;                          // sin(r + q pi/2), cos(r + q pi/2)
  const float cv = (q & 1) ? sr : cr;
  *s = (q & 2) ? -sv : sv;
  *c = ((q + 1) & 2) ? -cv : cv;
}

}  // namespace rel

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

}  // namespace rel

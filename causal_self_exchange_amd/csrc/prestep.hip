// Model-side pre-steps of Multi-Head Relation in one HBM pass: rotary
// position encoding of the relation coordinates P1 and P2 (full head, base
// configurable, [paper] App. B.3) and Givens mixing of the information heads
// in adjacent pairs ([paper] Eq. (4), App. A.2.2-A.2.3), where [paper] is
// "Ask Self, Ask Others: Relation Is All You Need".
//
// One thread per (b, h, t, group of 8 rotary pairs): it loads 16 elements of
// P1 and of P2, rotates them with the same 8 angles and stores them; if h is
// the first head of its Givens pair it also mixes the pair's 16 information
// elements at the same (b, t) and stores both heads. A thread issues all of
// its loads before its first store (one memory round trip), and every output
// element is written by the thread that read its inputs, so the outputs may
// be the inputs (in place).
//
// Rotary pair k (k = 0 .. d_h/2 - 1) turns by pos * base^(-2k/d_h):
//   interleaved: (x_{2k}, x_{2k+1});   half: (x_k, x_{k + d_h/2}).
// The angle is formed and reduced in fp64 before the fp32 sine and cosine,
// so positions in the thousands keep full fp32 accuracy.
#include "rel_internal.h"
#include "rel_device.h"

namespace rel {

namespace {

constexpr int kThreads = 256;

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

template <typename Tin>
__device__ __forceinline__ void store8(Tin* p, const float (&x)[8]) {
  if constexpr (sizeof(Tin) == 2) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8*>(p) = v;
  } else {
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// Rotate 8 pairs (a[e], b[e]) by angles with cosines c[e], sines s[e].
__device__ __forceinline__ void rotate(float (&a)[8], float (&b)[8], const float (&c)[8], const float (&s)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = a[e], y = b[e];
    a[e] = fmaf(x, c[e], -y * s[e]);
    b[e] = fmaf(x, s[e], y * c[e]);
  }
}

template <typename Tin, int D>
__global__ __launch_bounds__(kThreads) void prestep_kernel(PrestepArgs a, PrestepParams pp) {
  constexpr int kGroups = D / 16;                    // groups of 8 rotary pairs per row
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long total = (long long)a.B * a.H * a.T * kGroups;
  if (idx >= total) return;
  const int g = (int)(idx % kGroups);
  const long long row = idx / kGroups;               // (b, h, t) row index
  const int t = (int)(row % a.T);
  const int h = (int)((row / a.T) % a.H);
  const int b = (int)(row / ((long long)a.T * a.H));
  const size_t ro = (size_t)row * D;

  // Every load of the thread is issued before its first store, so one memory
  // round trip covers it (in place, each element is stored by the thread
  // that loaded it).
  // Coordinates: the two 8-element halves of this group's 8 rotary pairs.
  //   interleaved: elements 16 g .. 16 g + 15;  half: 8 g .. +7 and d/2 + 8 g .. +7.
  const int oa = a.rope == 2 ? 8 * g : 16 * g;
  const int ob = a.rope == 2 ? D / 2 + 8 * g : 16 * g + 8;
  const bool copy_coords = a.rope != 0 || a.P1o != a.P1 || a.P2o != a.P2;
  float c1[2][8], c2[2][8];                          // [half][element] of P1 and P2
  if (copy_coords) {
    const Tin* P1 = static_cast<const Tin*>(a.P1) + ro;
    const Tin* P2 = static_cast<const Tin*>(a.P2) + ro;
    if (!a.skip_p1) {
      load8(P1 + oa, c1[0]);
      load8(P1 + ob, c1[1]);
    }
    load8(P2 + oa, c2[0]);
    load8(P2 + ob, c2[1]);
  }
  // Information heads: this head's 16 elements, and its partner's when it
  // leads a Givens pair (pairing A: (2p, 2p+1); pairing B: (2p+1, (2p+2) mod H)).
  const Tin* I = static_cast<const Tin*>(a.I);
  Tin* Io = static_cast<Tin*>(a.Io);
  const bool lead = a.mix && (a.pairing == 0 ? (h % 2 == 0) : (h % 2 == 1));
  const bool copy_info = a.mix ? lead : Io != I;
  const int partner = a.pairing == 0 ? h + 1 : (h + 1) % a.H;
  const size_t ra = ro + 16 * g;
  const size_t rb = (((size_t)b * a.H + partner) * a.T + t) * D + 16 * g;
  float xi[2][8], yi[2][8];
  if (copy_info) {
    load8(I + ra, xi[0]);
    load8(I + ra + 8, xi[1]);
    if (lead) {
      load8(I + rb, yi[0]);
      load8(I + rb + 8, yi[1]);
    }
  }

  if (a.rope != 0) {
    const long long pos = (long long)(a.pos0 ? a.pos0[b] : 0) + t;
    float c[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sincos_of((double)pos * pp.inv_freq[8 * g + e], &sn[e], &c[e]);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      if (w == 0 && a.skip_p1) continue;
      float(&x)[2][8] = w ? c2 : c1;
      if (a.rope == 1) {
        // pairs (x0,x1) (x2,x3) ... of the 16 consecutive elements
        float p[8], q[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = x[0][2 * e]; q[e] = x[0][2 * e + 1];
          p[4 + e] = x[1][2 * e]; q[4 + e] = x[1][2 * e + 1];
        }
        rotate(p, q, c, sn);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[0][2 * e] = p[e]; x[0][2 * e + 1] = q[e];
          x[1][2 * e] = p[4 + e]; x[1][2 * e + 1] = q[4 + e];
        }
      } else {
        rotate(x[0], x[1], c, sn);
      }
    }
  }
  if (copy_coords) {
    Tin* P1o = static_cast<Tin*>(a.P1o) + ro;
    Tin* P2o = static_cast<Tin*>(a.P2o) + ro;
    if (!a.skip_p1) {
      store8(P1o + oa, c1[0]);
      store8(P1o + ob, c1[1]);
    }
    store8(P2o + oa, c2[0]);
    store8(P2o + ob, c2[1]);
  }

  if (copy_info) {
    if (lead) {
      const int pr = a.pairing == 0 ? h / 2 : (h - 1) / 2;
      const float ct = pp.cos_theta[pr], st = pp.sin_theta[pr];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float u = xi[half][e], v = yi[half][e];
          xi[half][e] = fmaf(ct, u, -st * v);
          yi[half][e] = fmaf(st, u, ct * v);
        }
      store8(Io + rb, yi[0]);
      store8(Io + rb + 8, yi[1]);
    }
    store8(Io + ra, xi[0]);
    store8(Io + ra + 8, xi[1]);
  }
}

template <typename Tin, int D>
hipError_t launch_typed(const PrestepArgs& a, const PrestepParams& pp, hipStream_t s) {
  const long long total = (long long)a.B * a.H * a.T * (D / 16);
  const long long blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prestep_kernel<Tin, D>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a, pp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prestep(const PrestepArgs& a, const PrestepParams& pp, bool bf16, hipStream_t s) {
  switch (a.d_h) {
    case 32: return bf16 ? launch_typed<__bf16, 32>(a, pp, s) : launch_typed<float, 32>(a, pp, s);
    case 48: return bf16 ? launch_typed<__bf16, 48>(a, pp, s) : launch_typed<float, 48>(a, pp, s);
    case 64: return bf16 ? launch_typed<__bf16, 64>(a, pp, s) : launch_typed<float, 64>(a, pp, s);
    case 80: return bf16 ? launch_typed<__bf16, 80>(a, pp, s) : launch_typed<float, 80>(a, pp, s);
    case 128: return bf16 ? launch_typed<__bf16, 128>(a, pp, s) : launch_typed<float, 128>(a, pp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rel

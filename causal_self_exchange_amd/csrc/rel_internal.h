// Internal declarations shared by the host API and the HIP kernel files of
// librelation.so. Not part of the public ABI (that is include/relation.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rel {

// Per-head reciprocal Self temperatures and the scalars every launch needs,
// passed by value in the kernel arguments (no device allocation).
struct HeadParams {
  float inv_tau[256];   // 1 / tau_h
  float scale;          // 1 / sqrt(d_h)
  float lambda;         // count-calibration coefficient
};

struct FwdArgs {
  const void* P1;
  const void* P2;
  const void* V;
  void* Y;
  int B, H, T, d_h;
};

struct DecodeArgs {
  const void* p1;
  const void* p2;
  const void* v;
  const void* cP2;
  const void* cV;
  const int32_t* len;
  void* y;
  float* ws;            // partial states [B][H][n_chunks][d_h + 2]
  int B, H, L_cap, d_h, n_chunks;
};

// Cache rows per decode partial state: the workspace holds ceil(L_cap / 256)
// states per (b, h), one per partial work-group.
constexpr int kDecodeChunk = 256;

// Launchers (return the hipError_t of the launch).
hipError_t launch_fwd_scan(const FwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
hipError_t launch_fwd_mfma_bf16(const FwdArgs& a, const HeadParams& hp, hipStream_t s);
bool fwd_mfma_supported(int d_h, int T);
hipError_t launch_decode(const DecodeArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
hipError_t launch_cache_append(void* cP2, void* cV, int32_t* len, const void* p2, const void* v,
                               int B, int H, int L_cap, int d_h, bool bf16, hipStream_t s);

}  // namespace rel

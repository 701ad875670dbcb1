// Internal declarations shared by the host API and the HIP kernel files of
// librelation.so. Not part of the public ABI (that is include/relation.h).
#pragma once

#include <hip/hip_runtime.h>

#include "relation.h"
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
  float* lse;           // optional [B][H][T] row log normalisers (null: not written)
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

// Backward of the forward above. Row statistics are stored per 64-row tile
// of each (b, h) as four arrays of 64 floats, so that one 1 KB direct load
// brings a tile's values into LDS:
//   [0]  (LSE_i + lambda log i) log2 e   (+inf on padding rows past T)
//   [1]  -D_i,  D_i = dY_i . Y_i
//   [2]  F_ii  (the Self weight of row i)
//   [3]  dU_ii / sqrt(d_h)  (Self gradient of the evidence, scaled)
// Partials of dtau / dlambda are written per (b, h, 256-row chunk) and summed
// in a fixed order by the reduce kernel, so every output is deterministic.
constexpr int kStatRows = 64;
constexpr int kStatTile = 4 * kStatRows;   // floats per 64-row tile of statistics
constexpr int kPrepRows = 256;             // rows per prep work-group (one partial)

struct BwdArgs {
  const void* P1;
  const void* P2;
  const void* V;
  const void* Y;
  const void* dY;
  const float* lse;     // [B][H][T] natural-log row normalisers from the forward
  void* dP1;
  void* dP2;
  void* dV;
  float* dtau;          // [H]
  float* dlambda;       // [1]
  float* stats;         // [B*H][ceil(T/64)][4][64]
  float* part;          // [B*H][ceil(T/256)][2]
  void* du;             // stored dU blocks (bf16 MFMA backward only), or null to recompute
  int B, H, T, d_h;
};

inline int64_t bwd_stat_floats(int64_t BH, int64_t T) { return BH * ((T + kStatRows - 1) / kStatRows) * kStatTile; }
inline int64_t bwd_part_floats(int64_t BH, int64_t T) { return BH * ((T + kPrepRows - 1) / kPrepRows) * 2; }

// Stored dU of the bf16 MFMA backward: per head, blocks of 32 queries x 16
// keys (1 KB of bf16) for every 32-query block qp and 16-key block kb with
// kb <= 2 qp + 1 (the lower triangle, strictly-causal entries; zeros above the
// diagonal), block (qp, kb) at index qp (qp + 1) + kb.
constexpr int kDuBlockBytes = 1024;
__host__ __device__ inline int64_t bwd_du_head_blocks(int64_t T) {
  const int64_t nqp = (T + 31) / 32;
  return nqp * (nqp + 1);
}
__host__ __device__ inline int64_t bwd_du_head_bytes(int64_t T) { return bwd_du_head_blocks(T) * kDuBlockBytes; }

// Model-side pre-steps: rotary encoding of P1 / P2 and Givens mixing of the
// information heads (one HBM pass; outputs may be the inputs).
struct PrestepArgs {
  const void* P1;
  const void* P2;
  const void* I;
  const int32_t* pos0;  // optional device int32[B]: position of row 0 per sequence
  void* P1o;
  void* P2o;
  void* Io;
  int B, H, T, d_h;
  int rope;             // 0 none, 1 interleaved pairs, 2 half split
  int pairing;          // 0: (1,2),(3,4),...; 1: (2,3),...,(H,1) (one-based heads)
  int mix;              // 1: Givens mixing of I, 0: copy
  int skip_p1;          // 1: P1 is neither read nor written (the forward rotates it)
};

struct PrestepParams {
  double inv_freq[64];  // base^(-2k/d_h), k < d_h / 2
  float cos_theta[128]; // per Givens pair
  float sin_theta[128];
};

// Linear Relation forward (chunk-parallel recurrence).
constexpr int kLinChunk = 64;          // tokens per chunk
struct LinArgs {
  const void* P1;
  const void* P2;
  const void* I;
  const float* alpha;   // [B][H][T][d_h] channel-wise retention
  void* Y;
  float* final;         // optional [B][H][d_h][d_h] final state C_T
  float* state;         // workspace: [B*H][groups][d_h][d_h] group states
  float* decay;         // workspace: [B*H][groups][d_h] group decays
  float* rowsc;         // workspace: [B*H][T][2] row factors S_t / |p1_t|, S_t / |p2_t|
  int B, H, T, d_h;
  int group;            // chunks per group (set by the launcher; groups = ceil(ceil(T/64) / group))
};
inline int64_t lin_state_floats(int64_t BH, int64_t T, int64_t D) { return BH * ((T + kLinChunk - 1) / kLinChunk) * D * D; }
inline int64_t lin_decay_floats(int64_t BH, int64_t T, int64_t D) { return BH * ((T + kLinChunk - 1) / kLinChunk) * D; }
inline int64_t lin_rowsc_floats(int64_t BH, int64_t T) { return BH * T * 2; }

// Cache rows per decode partial state: the workspace holds ceil(L_cap / 256)
// states per (b, h), one per partial work-group.
constexpr int kDecodeChunk = 256;
// Size of the device array that holds relation_decode_noalloc's partial
// states (B * H * ceil(L_cap / 256) * (d_h + 2) floats must fit).
constexpr size_t kDecodeScratchBytes = REL_DECODE_SCRATCH_BYTES;

// Launchers (return the hipError_t of the launch).
hipError_t launch_fwd_scan(const FwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
// Compute units of the current device (queried once per device, then cached:
// the library's only global state).
hipError_t device_cu_count(int* n_cu);
// Rotary encoding of P1 applied by the MFMA forward as it loads a query tile
// (relation_fwd_model): the pre-step's rotation of each row, with the same
// angles and roundings, so the result equals pre-step then forward.
struct RopeParams {
  const int32_t* pos0;  // optional device int32[B]: position of row 0 per sequence
  int rope;             // 1 interleaved pairs, 2 half split
  double inv_freq[64];  // base^(-2k/d_h), k < d_h / 2
};
hipError_t launch_fwd_mfma_bf16(const FwdArgs& a, const HeadParams& hp, hipStream_t s,
                                const RopeParams* rope = nullptr);
bool fwd_mfma_supported(int d_h, int T);
// Whether the MFMA forward can rotate P1 itself: interleaved pairs at any
// head size, half-split pairs where both halves of a pair sit in one lane
// (d_h a multiple of 32).
bool fwd_mfma_rope_fusable(int d_h, int rope);
// Backward: prep (row statistics, dtau / dlambda partials) then the query and
// key/value gradient kernels, then the fixed-order reduce.
hipError_t launch_bwd_prep(const BwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
hipError_t launch_bwd_scan(const BwdArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
hipError_t launch_bwd_mfma_bf16(const BwdArgs& a, const HeadParams& hp, hipStream_t s);
hipError_t launch_bwd_reduce(const BwdArgs& a, hipStream_t s);
bool bwd_mfma_supported(int d_h, int T);
// Whether the bf16 MFMA backward can store dU for this length (one head's
// blocks addressed with 31-bit byte offsets).
bool bwd_du_supported(int d_h, int T);
hipError_t launch_prestep(const PrestepArgs& a, const PrestepParams& pp, bool bf16, hipStream_t s);
hipError_t launch_linear(const LinArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, const HeadParams& hp, bool bf16, hipStream_t s);
// Device address of the decode scratch array on the current device.
hipError_t decode_scratch(void** ptr);
hipError_t launch_cache_append(void* cP2, void* cV, int32_t* len, const void* p2, const void* v,
                               int B, int H, int L_cap, int d_h, bool bf16, hipStream_t s);

}  // namespace rel

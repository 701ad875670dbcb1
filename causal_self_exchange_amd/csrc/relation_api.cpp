// Host side of librelation.so: argument validation, per-head parameter
// packing and kernel dispatch for the C ABI declared in include/relation.h.
// Every check runs before any HIP call, so an invalid call launches nothing.
#include "relation.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "rel_internal.h"

namespace {

using rel::HeadParams;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t elem_size(rel_dtype dt) { return dt == REL_BF16 ? 2 : 4; }

bool dtype_ok(rel_dtype dt) { return dt == REL_F32 || dt == REL_BF16; }

bool head_dim_ok(int d_h) { return d_h == 32 || d_h == 64 || d_h == 128; }
// The forward, its training variant, the backward and the pre-steps also take
// the paper's non-power-of-two head sizes.
bool fwd_head_dim_ok(int d_h) { return head_dim_ok(d_h) || d_h == 48 || d_h == 80; }

// Product of positive ints; false if any is < 1 or the product exceeds 2^40
// elements (4 TiB of fp32, far beyond one GPU's memory).
bool count(int64_t& out, std::initializer_list<int64_t> dims) {
  constexpr int64_t kMaxElems = int64_t(1) << 40;
  int64_t p = 1;
  for (int64_t d : dims) {
    if (d < 1) return false;
    if (p > kMaxElems / d) return false;
    p *= d;
  }
  out = p;
  return true;
}

rel_status pack_heads(HeadParams& hp, const float* tau, int H, int d_h, float lambda) {
  if (!std::isfinite(lambda)) return REL_E_LAMBDA;
  for (int h = 0; h < H; ++h) {
    const float t = tau[h];
    if (!std::isfinite(t) || !(t > 0.0f)) return REL_E_TAU;
    hp.inv_tau[h] = 1.0f / t;
  }
  for (int h = H; h < REL_MAX_HEADS; ++h) hp.inv_tau[h] = 0.0f;
  hp.scale = 1.0f / std::sqrt(static_cast<float>(d_h));
  hp.lambda = lambda;
  return REL_OK;
}

// Kernel selection (relation_select_kernels): process-wide, initialised once
// from RELATION_FWD_KERNEL / RELATION_BWD_KERNEL.
std::atomic<int> g_fwd_kernel{REL_KERNEL_AUTO}, g_bwd_kernel{REL_KERNEL_AUTO};
std::once_flag g_kernel_env_once;

void read_kernel_env() {
  std::call_once(g_kernel_env_once, [] {
    auto scan = [](const char* name) {
      const char* v = std::getenv(name);
      return v && std::strcmp(v, "scan") == 0;
    };
    if (scan("RELATION_FWD_KERNEL")) g_fwd_kernel.store(REL_KERNEL_SCAN, std::memory_order_relaxed);
    if (scan("RELATION_BWD_KERNEL")) g_bwd_kernel.store(REL_KERNEL_SCAN, std::memory_order_relaxed);
  });
}

// Which forward kernel runs: the MFMA kernel for bf16 where it exists, else
// the row-scan kernel (always, once REL_KERNEL_SCAN is selected).
bool use_mfma(rel_dtype dt, int d_h, int T) {
  if (dt != REL_BF16 || !rel::fwd_mfma_supported(d_h, T)) return false;
  read_kernel_env();
  return g_fwd_kernel.load(std::memory_order_relaxed) != REL_KERNEL_SCAN;
}

// Forward with an optional row log-normaliser output (lse may be null).
rel_status fwd_impl(const void* P1, const void* P2, const void* V, const float* tau_s, float lambda,
                    void* Y, float* lse, int B, int H, int T, int d_h, rel_dtype dt, hipStream_t stream) {
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || H > REL_MAX_HEADS || B > 65535) return REL_E_SHAPE;
  if (!dtype_ok(dt)) return REL_E_DTYPE;
  if (!fwd_head_dim_ok(d_h)) return REL_E_HEADDIM;
  HeadParams hp;
  const rel_status st = pack_heads(hp, tau_s, H, d_h, lambda);
  if (st != REL_OK) return st;
  if (!aligned16(P1) || !aligned16(P2) || !aligned16(V) || !aligned16(Y)) return REL_E_ALIGN;
  const size_t bytes = static_cast<size_t>(n) * elem_size(dt);
  if (overlaps(Y, bytes, P1, bytes) || overlaps(Y, bytes, P2, bytes) || overlaps(Y, bytes, V, bytes))
    return REL_E_ALIAS;
  if (lse) {
    if (!aligned4(lse)) return REL_E_ALIGN;
    const size_t lb = static_cast<size_t>(B) * H * T * sizeof(float);
    if (overlaps(lse, lb, P1, bytes) || overlaps(lse, lb, P2, bytes) || overlaps(lse, lb, V, bytes) ||
        overlaps(lse, lb, Y, bytes))
      return REL_E_ALIAS;
  }

  rel::FwdArgs a{P1, P2, V, Y, B, H, T, d_h, lse};
  const hipError_t e = use_mfma(dt, d_h, T) ? rel::launch_fwd_mfma_bf16(a, hp, stream)
                                         : rel::launch_fwd_scan(a, hp, dt == REL_BF16, stream);
  return e == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

// Which backward runs: the MFMA kernels for bf16 where they exist, else the
// row-scan kernels (always, once REL_KERNEL_SCAN is selected).
bool use_bwd_mfma(rel_dtype dt, int d_h, int T) {
  if (dt != REL_BF16 || !rel::bwd_mfma_supported(d_h, T)) return false;
  read_kernel_env();
  return g_bwd_kernel.load(std::memory_order_relaxed) != REL_KERNEL_SCAN;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Validates a pre-step call and fills its launch arguments (no HIP call).
rel_status prestep_setup(rel::PrestepArgs& a, rel::PrestepParams& pp, const void* P1, const void* P2,
                         const void* I, const int32_t* pos0, rel_rope rope, float rope_base,
                         const float* theta, rel_pairing pairing, void* P1o, void* P2o, void* Io, int B,
                         int H, int T, int d_h, rel_dtype dt) {
  if (!P1 || !P2 || !I || !P1o || !P2o || !Io) return REL_E_NULL;
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || H > REL_MAX_HEADS || B > 65535) return REL_E_SHAPE;
  if (theta && (H % 2 != 0)) return REL_E_SHAPE;
  if (!dtype_ok(dt)) return REL_E_DTYPE;
  if (!fwd_head_dim_ok(d_h)) return REL_E_HEADDIM;
  if (rope != REL_ROPE_NONE && rope != REL_ROPE_INTERLEAVED && rope != REL_ROPE_HALF) return REL_E_PRESTEP;
  if (pairing != REL_PAIRS_A && pairing != REL_PAIRS_B) return REL_E_PRESTEP;
  if (rope != REL_ROPE_NONE && !(std::isfinite(rope_base) && rope_base > 1.0f)) return REL_E_PRESTEP;
  if (theta)
    for (int k = 0; k < H / 2; ++k)
      if (!std::isfinite(theta[k])) return REL_E_PRESTEP;
  if (!aligned16(P1) || !aligned16(P2) || !aligned16(I) || !aligned16(P1o) || !aligned16(P2o) ||
      !aligned16(Io) || (reinterpret_cast<uintptr_t>(pos0) & 3u))
    return REL_E_ALIGN;
  const size_t tb = static_cast<size_t>(n) * elem_size(dt);
  const size_t pb = static_cast<size_t>(B) * sizeof(int32_t);
  // Each output may be its own input (in place) but may overlap nothing else.
  const void* ins[3] = {P1, P2, I};
  void* outs[3] = {P1o, P2o, Io};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 3; ++i)
      if (!(o == i && outs[o] == ins[i]) && overlaps(outs[o], tb, ins[i], tb)) return REL_E_ALIAS;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(outs[o], tb, outs[q], tb)) return REL_E_ALIAS;
    if (pos0 && overlaps(outs[o], tb, pos0, pb)) return REL_E_ALIAS;
  }
  a = rel::PrestepArgs{P1, P2, I, pos0, P1o, P2o, Io, B, H, T, d_h, static_cast<int>(rope),
                       pairing == REL_PAIRS_A ? 0 : 1, theta ? 1 : 0};
  for (int k = 0; k < 64; ++k)
    pp.inv_freq[k] = k < d_h / 2 ? std::pow(static_cast<double>(rope_base), -2.0 * k / d_h) : 0.0;
  for (int k = 0; k < 128; ++k) {
    const double t = (theta && k < H / 2) ? static_cast<double>(theta[k]) : 0.0;
    pp.cos_theta[k] = static_cast<float>(std::cos(t));
    pp.sin_theta[k] = static_cast<float>(std::sin(t));
  }
  return REL_OK;
}

}  // namespace

extern "C" {

const char* relation_status_str(rel_status s) {
  switch (s) {
    case REL_OK: return "ok";
    case REL_E_NULL: return "null pointer";
    case REL_E_SHAPE: return "invalid shape";
    case REL_E_DTYPE: return "unknown dtype";
    case REL_E_HEADDIM: return "unsupported head dimension";
    case REL_E_TAU: return "tau must be finite and > 0";
    case REL_E_LAMBDA: return "lambda must be finite";
    case REL_E_ALIGN: return "pointer misaligned (16 bytes; 4 for float arrays)";
    case REL_E_ALIAS: return "output overlaps an input or another output";
    case REL_E_WORKSPACE: return "workspace missing or too small";
    case REL_E_LAUNCH: return "kernel launch failed";
    case REL_E_PRESTEP: return "invalid rotary mode, base, pairing or Givens angle";
    case REL_E_KERNEL: return "unknown kernel selection";
  }
  return "unknown status";
}

rel_status relation_fwd_ex(const void* P1, const void* P2, const void* V, const float* tau_s,
                           float lambda, void* Y, int B, int H, int T, int d_h, rel_dtype dt,
                           hipStream_t stream) {
  if (!P1 || !P2 || !V || !tau_s || !Y) return REL_E_NULL;
  return fwd_impl(P1, P2, V, tau_s, lambda, Y, nullptr, B, H, T, d_h, dt, stream);
}

rel_status relation_fwd_lse(const void* P1, const void* P2, const void* V, const float* tau_s,
                            float lambda, void* Y, float* LSE, int B, int H, int T, int d_h,
                            rel_dtype dt, hipStream_t stream) {
  if (!P1 || !P2 || !V || !tau_s || !Y || !LSE) return REL_E_NULL;
  return fwd_impl(P1, P2, V, tau_s, lambda, Y, LSE, B, H, T, d_h, dt, stream);
}

rel_status relation_prestep(const void* P1, const void* P2, const void* I, const int32_t* pos0,
                            rel_rope rope, float rope_base, const float* theta, rel_pairing pairing,
                            void* P1o, void* P2o, void* Io, int B, int H, int T, int d_h, rel_dtype dt,
                            hipStream_t stream) {
  rel::PrestepArgs a;
  rel::PrestepParams pp;
  const rel_status st = prestep_setup(a, pp, P1, P2, I, pos0, rope, rope_base, theta, pairing, P1o, P2o, Io,
                                      B, H, T, d_h, dt);
  if (st != REL_OK) return st;
  return rel::launch_prestep(a, pp, dt == REL_BF16, stream) == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

size_t relation_fwd_model_workspace_bytes(int B, int H, int T, int d_h, rel_dtype dt) {
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || !fwd_head_dim_ok(d_h) || !dtype_ok(dt)) return 0;
  return 3 * align256(static_cast<size_t>(n) * elem_size(dt));
}

rel_status relation_fwd_model(const void* P1, const void* P2, const void* I, const int32_t* pos0,
                              rel_rope rope, float rope_base, const float* theta, rel_pairing pairing,
                              const float* tau_s, float lambda, void* Y, float* LSE, int B, int H, int T,
                              int d_h, rel_dtype dt, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!P1 || !P2 || !I || !tau_s || !Y) return REL_E_NULL;
  const size_t need = relation_fwd_model_workspace_bytes(B, H, T, d_h, dt);
  if (need == 0) {
    int64_t n = 0;
    if (!count(n, {B, H, T, d_h})) return REL_E_SHAPE;
    return dtype_ok(dt) ? REL_E_HEADDIM : REL_E_DTYPE;
  }
  if (!workspace || ws_bytes < need) return REL_E_WORKSPACE;
  if (H > REL_MAX_HEADS || B > 65535) return REL_E_SHAPE;
  const size_t part = need / 3;
  char* ws = static_cast<char*>(workspace);
  rel::PrestepArgs a;
  rel::PrestepParams pp;
  rel_status st = prestep_setup(a, pp, P1, P2, I, pos0, rope, rope_base, theta, pairing, ws, ws + part,
                                ws + 2 * part, B, H, T, d_h, dt);
  if (st != REL_OK) return st;
  // The forward's own checks (tau, lambda, Y and LSE against the workspace
  // tensors and the raw inputs) run before anything is launched.
  const size_t tb = static_cast<size_t>(B) * H * T * d_h * elem_size(dt);
  if (!aligned16(Y)) return REL_E_ALIGN;
  if (overlaps(Y, tb, P1, tb) || overlaps(Y, tb, P2, tb) || overlaps(Y, tb, I, tb) ||
      overlaps(Y, tb, workspace, need) || (pos0 && overlaps(Y, tb, pos0, static_cast<size_t>(B) * 4)))
    return REL_E_ALIAS;
  if (LSE) {
    const size_t lb = static_cast<size_t>(B) * H * T * sizeof(float);
    if (!aligned4(LSE)) return REL_E_ALIGN;
    if (overlaps(LSE, lb, P1, tb) || overlaps(LSE, lb, P2, tb) || overlaps(LSE, lb, I, tb) ||
        overlaps(LSE, lb, Y, tb) || overlaps(LSE, lb, workspace, need) ||
        (pos0 && overlaps(LSE, lb, pos0, static_cast<size_t>(B) * 4)))
      return REL_E_ALIAS;
  }
  HeadParams hp;
  st = pack_heads(hp, tau_s, H, d_h, lambda);
  if (st != REL_OK) return st;
  // The bf16 MFMA forward rotates P1 itself as it loads each query tile: the
  // pre-step then rotates P2 and mixes I only, and P1 is read once.
  const bool fuse = rope != REL_ROPE_NONE && use_mfma(dt, d_h, T) &&
                    rel::fwd_mfma_rope_fusable(d_h, static_cast<int>(rope));
  if (fuse) a.skip_p1 = 1;
  if (rel::launch_prestep(a, pp, dt == REL_BF16, stream) != hipSuccess) return REL_E_LAUNCH;
  if (!fuse) return fwd_impl(ws, ws + part, ws + 2 * part, tau_s, lambda, Y, LSE, B, H, T, d_h, dt, stream);
  rel::RopeParams rp;
  rp.pos0 = pos0;
  rp.rope = static_cast<int>(rope);
  for (int k = 0; k < 64; ++k) rp.inv_freq[k] = pp.inv_freq[k];
  const rel::FwdArgs fa{P1, ws + part, ws + 2 * part, Y, B, H, T, d_h, LSE};
  return rel::launch_fwd_mfma_bf16(fa, hp, stream, &rp) == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

size_t relation_linear_workspace_bytes(int B, int H, int T, int d_h) {
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || !head_dim_ok(d_h)) return 0;
  const int64_t BH = static_cast<int64_t>(B) * H;
  return align256(static_cast<size_t>(rel::lin_state_floats(BH, T, d_h)) * sizeof(float)) +
         align256(static_cast<size_t>(rel::lin_decay_floats(BH, T, d_h)) * sizeof(float)) +
         align256(static_cast<size_t>(rel::lin_rowsc_floats(BH, T)) * sizeof(float));
}

rel_status relation_linear_fwd(const void* P1, const void* P2, const void* I, const float* alpha,
                               const float* tau_s, void* Y, float* state_out, int B, int H, int T, int d_h,
                               rel_dtype dt, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!P1 || !P2 || !I || !alpha || !tau_s || !Y) return REL_E_NULL;
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || H > REL_MAX_HEADS || B > 65535) return REL_E_SHAPE;
  if (!dtype_ok(dt)) return REL_E_DTYPE;
  if (!head_dim_ok(d_h)) return REL_E_HEADDIM;
  HeadParams hp;
  const rel_status st = pack_heads(hp, tau_s, H, d_h, 0.0f);
  if (st != REL_OK) return st;
  const size_t need = relation_linear_workspace_bytes(B, H, T, d_h);
  if (!workspace || ws_bytes < need) return REL_E_WORKSPACE;
  if (!aligned16(P1) || !aligned16(P2) || !aligned16(I) || !aligned16(Y) || !aligned16(alpha) ||
      !aligned16(workspace) || !aligned16(state_out))
    return REL_E_ALIGN;
  const size_t tb = static_cast<size_t>(n) * elem_size(dt);
  const size_t ab = static_cast<size_t>(n) * sizeof(float);
  const size_t sb = static_cast<size_t>(B) * H * d_h * d_h * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range ins[] = {{P1, tb}, {P2, tb}, {I, tb}, {alpha, ab}};
  const Range outs[] = {{Y, tb}, {state_out, state_out ? sb : 0}, {workspace, need}};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (o.n && overlaps(o.p, o.n, i.p, i.n)) return REL_E_ALIAS;
  for (size_t x = 0; x < 3; ++x)
    for (size_t y = x + 1; y < 3; ++y)
      if (outs[x].n && outs[y].n && overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return REL_E_ALIAS;

  const int64_t BH = static_cast<int64_t>(B) * H;
  char* ws = static_cast<char*>(workspace);
  float* state = reinterpret_cast<float*>(ws);
  const size_t state_bytes = align256(static_cast<size_t>(rel::lin_state_floats(BH, T, d_h)) * sizeof(float));
  const size_t decay_bytes = align256(static_cast<size_t>(rel::lin_decay_floats(BH, T, d_h)) * sizeof(float));
  float* decay = reinterpret_cast<float*>(ws + state_bytes);
  float* rowsc = reinterpret_cast<float*>(ws + state_bytes + decay_bytes);
  rel::LinArgs a{P1, P2, I, alpha, Y, state_out, state, decay, rowsc, B, H, T, d_h, 1};
  return rel::launch_linear(a, hp, dt == REL_BF16, stream) == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

size_t relation_bwd_workspace_bytes(int B, int H, int T, int d_h) {
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || !fwd_head_dim_ok(d_h)) return 0;
  const int64_t BH = static_cast<int64_t>(B) * H;
  return align256(static_cast<size_t>(rel::bwd_stat_floats(BH, T)) * sizeof(float)) +
         align256(static_cast<size_t>(rel::bwd_part_floats(BH, T)) * sizeof(float));
}

size_t relation_bwd_stored_workspace_bytes(int B, int H, int T, int d_h) {
  const size_t base = relation_bwd_workspace_bytes(B, H, T, d_h);
  if (base == 0 || !rel::bwd_du_supported(d_h, T)) return 0;
  const int64_t BH = static_cast<int64_t>(B) * H;
  const int64_t hb = rel::bwd_du_head_bytes(T);
  if (BH > (INT64_MAX / 2) / hb) return 0;
  return base + align256(static_cast<size_t>(BH * hb));
}

rel_status relation_bwd(const void* P1, const void* P2, const void* V, const float* tau_s,
                        float lambda, const void* Y, const float* LSE, const void* dY, void* dP1,
                        void* dP2, void* dV, float* dtau, float* dlambda, int B, int H, int T,
                        int d_h, rel_dtype dt, void* workspace, size_t ws_bytes,
                        hipStream_t stream) {
  if (!P1 || !P2 || !V || !tau_s || !Y || !LSE || !dY || !dP1 || !dP2 || !dV || !dtau || !dlambda)
    return REL_E_NULL;
  int64_t n = 0;
  if (!count(n, {B, H, T, d_h}) || H > REL_MAX_HEADS || B > 65535) return REL_E_SHAPE;
  if (!dtype_ok(dt)) return REL_E_DTYPE;
  if (!fwd_head_dim_ok(d_h)) return REL_E_HEADDIM;
  HeadParams hp;
  const rel_status st = pack_heads(hp, tau_s, H, d_h, lambda);
  if (st != REL_OK) return st;
  const size_t base = relation_bwd_workspace_bytes(B, H, T, d_h);
  if (!workspace || ws_bytes < base) return REL_E_WORKSPACE;
  // The bf16 MFMA backward stores dU when the workspace holds it.
  const size_t stored = relation_bwd_stored_workspace_bytes(B, H, T, d_h);
  const bool mfma = use_bwd_mfma(dt, d_h, T);
  const bool store_du = mfma && stored != 0 && ws_bytes >= stored;
  const size_t need = store_du ? stored : base;
  if (!aligned16(P1) || !aligned16(P2) || !aligned16(V) || !aligned16(Y) || !aligned16(dY) ||
      !aligned16(dP1) || !aligned16(dP2) || !aligned16(dV) || !aligned16(workspace) || !aligned4(LSE) ||
      !aligned4(dtau) || !aligned4(dlambda))
    return REL_E_ALIGN;
  const size_t tb = static_cast<size_t>(n) * elem_size(dt);
  const size_t lb = static_cast<size_t>(B) * H * T * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range ins[] = {{P1, tb}, {P2, tb}, {V, tb}, {Y, tb}, {LSE, lb}, {dY, tb}};
  const Range outs[] = {{dP1, tb}, {dP2, tb}, {dV, tb}, {dtau, H * sizeof(float)},
                        {dlambda, sizeof(float)}, {workspace, need}};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return REL_E_ALIAS;
  for (size_t x = 0; x < sizeof(outs) / sizeof(outs[0]); ++x)
    for (size_t y = x + 1; y < sizeof(outs) / sizeof(outs[0]); ++y)
      if (overlaps(outs[x].p, outs[x].n, outs[y].p, outs[y].n)) return REL_E_ALIAS;

  const int64_t BH = static_cast<int64_t>(B) * H;
  char* ws = static_cast<char*>(workspace);
  float* stats = reinterpret_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(ws + align256(static_cast<size_t>(rel::bwd_stat_floats(BH, T)) * sizeof(float)));
  void* du = store_du ? static_cast<void*>(ws + base) : nullptr;
  rel::BwdArgs a{P1, P2, V, Y, dY, LSE, dP1, dP2, dV, dtau, dlambda, stats, part, du, B, H, T, d_h};
  const bool bf16 = dt == REL_BF16;
  hipError_t e;
  if (mfma) {
    // Recomputing: the MFMA query kernel forms the row statistics itself.
    // Storing dU: the prep kernel forms them first.
    e = rel::launch_bwd_mfma_bf16(a, hp, stream);
  } else {
    e = rel::launch_bwd_prep(a, hp, bf16, stream);
    if (e == hipSuccess) e = rel::launch_bwd_scan(a, hp, bf16, stream);
  }
  if (e == hipSuccess) e = rel::launch_bwd_reduce(a, stream);
  return e == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

rel_status relation_fwd(const void* P1, const void* P2, const void* V, const float* tau_s, void* Y,
                        int B, int H, int T, int d_h, rel_dtype dt, hipStream_t stream) {
  return relation_fwd_ex(P1, P2, V, tau_s, 0.0f, Y, B, H, T, d_h, dt, stream);
}

size_t relation_decode_workspace_bytes(int B, int H, int L_cap, int d_h) {
  int64_t n = 0;
  if (!count(n, {B, H, L_cap, d_h}) || !fwd_head_dim_ok(d_h)) return 0;
  const int64_t chunks = (L_cap + rel::kDecodeChunk - 1) / rel::kDecodeChunk;
  return static_cast<size_t>(B) * H * chunks * (d_h + 2) * sizeof(float);
}

namespace {

// relation_decode with its workspace either passed in (scratch == false) or
// the library's scratch array (scratch == true; then `workspace` is unused).
rel_status decode_impl(const void* p1, const void* p2, const void* v, const void* cache_P2,
                       const void* cache_V, const int32_t* len, const float* tau_s, float lambda, void* y,
                       int B, int H, int L_cap, int d_h, rel_dtype dt, void* workspace, size_t ws_bytes,
                       bool scratch, hipStream_t stream) {
  if (!p1 || !p2 || !v || !cache_P2 || !cache_V || !len || !tau_s || !y) return REL_E_NULL;
  int64_t ncache = 0, ntok = 0;
  if (!count(ncache, {B, H, L_cap, d_h}) || !count(ntok, {B, H, d_h}) || H > REL_MAX_HEADS ||
      B > 65535)
    return REL_E_SHAPE;
  if (!dtype_ok(dt)) return REL_E_DTYPE;
  if (!fwd_head_dim_ok(d_h)) return REL_E_HEADDIM;
  HeadParams hp;
  const rel_status st = pack_heads(hp, tau_s, H, d_h, lambda);
  if (st != REL_OK) return st;
  const size_t need = relation_decode_workspace_bytes(B, H, L_cap, d_h);
  if (scratch) {
    // Every check above and below runs before the one HIP call that finds the
    // scratch array's address.
    if (need > rel::kDecodeScratchBytes) return REL_E_WORKSPACE;
  } else if (!workspace || ws_bytes < need) {
    return REL_E_WORKSPACE;
  }
  if (!aligned16(p1) || !aligned16(p2) || !aligned16(v) || !aligned16(cache_P2) ||
      !aligned16(cache_V) || !aligned16(y) || (!scratch && !aligned16(workspace)) ||
      (reinterpret_cast<uintptr_t>(len) & 3u))
    return REL_E_ALIGN;
  const size_t es = elem_size(dt);
  const size_t tb = static_cast<size_t>(ntok) * es, cb = static_cast<size_t>(ncache) * es;
  const size_t lb = static_cast<size_t>(B) * sizeof(int32_t);
  if (overlaps(y, tb, p1, tb) || overlaps(y, tb, p2, tb) || overlaps(y, tb, v, tb) ||
      overlaps(y, tb, cache_P2, cb) || overlaps(y, tb, cache_V, cb) || overlaps(y, tb, len, lb) ||
      (!scratch && overlaps(y, tb, workspace, need)))
    return REL_E_ALIAS;
  if (!scratch && (overlaps(workspace, need, p1, tb) || overlaps(workspace, need, p2, tb) ||
                   overlaps(workspace, need, v, tb) || overlaps(workspace, need, cache_P2, cb) ||
                   overlaps(workspace, need, cache_V, cb) || overlaps(workspace, need, len, lb)))
    return REL_E_ALIAS;
  if (scratch) {
    void* p = nullptr;
    if (rel::decode_scratch(&p) != hipSuccess) return REL_E_LAUNCH;
    workspace = p;
  }

  rel::DecodeArgs a{p1, p2, v, cache_P2, cache_V, len, y, static_cast<float*>(workspace),
                    B, H, L_cap, d_h, static_cast<int>((L_cap + rel::kDecodeChunk - 1) / rel::kDecodeChunk)};
  const hipError_t e = rel::launch_decode(a, hp, dt == REL_BF16, stream);
  return e == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

}  // namespace

rel_status relation_decode(const void* p1, const void* p2, const void* v, const void* cache_P2,
                           const void* cache_V, const int32_t* len, const float* tau_s, float lambda,
                           void* y, int B, int H, int L_cap, int d_h, rel_dtype dt, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  return decode_impl(p1, p2, v, cache_P2, cache_V, len, tau_s, lambda, y, B, H, L_cap, d_h, dt, workspace,
                     ws_bytes, false, stream);
}

rel_status relation_decode_noalloc(const void* p1, const void* p2, const void* v, const void* cache_P2,
                                   const void* cache_V, const int32_t* len, const float* tau_s, float lambda,
                                   void* y, int B, int H, int L_cap, int d_h, rel_dtype dt,
                                   hipStream_t stream) {
  return decode_impl(p1, p2, v, cache_P2, cache_V, len, tau_s, lambda, y, B, H, L_cap, d_h, dt, nullptr, 0,
                     true, stream);
}

rel_status relation_cache_append(void* cache_P2, void* cache_V, int32_t* len, const void* p2,
                                 const void* v, int B, int H, int L_cap, int d_h, rel_dtype dt,
                                 hipStream_t stream) {
  if (!cache_P2 || !cache_V || !len || !p2 || !v) return REL_E_NULL;
  int64_t ncache = 0, ntok = 0;
  if (!count(ncache, {B, H, L_cap, d_h}) || !count(ntok, {B, H, d_h}) || H > REL_MAX_HEADS ||
      B > 65535)
    return REL_E_SHAPE;
  if (!dtype_ok(dt)) return REL_E_DTYPE;
  if (!fwd_head_dim_ok(d_h)) return REL_E_HEADDIM;
  if (!aligned16(cache_P2) || !aligned16(cache_V) || !aligned16(p2) || !aligned16(v) ||
      (reinterpret_cast<uintptr_t>(len) & 3u))
    return REL_E_ALIGN;
  const size_t es = elem_size(dt);
  const size_t tb = static_cast<size_t>(ntok) * es, cb = static_cast<size_t>(ncache) * es;
  const size_t lb = static_cast<size_t>(B) * sizeof(int32_t);
  if (overlaps(cache_P2, cb, cache_V, cb) || overlaps(cache_P2, cb, p2, tb) ||
      overlaps(cache_P2, cb, v, tb) || overlaps(cache_V, cb, p2, tb) || overlaps(cache_V, cb, v, tb) ||
      overlaps(len, lb, cache_P2, cb) || overlaps(len, lb, cache_V, cb) || overlaps(len, lb, p2, tb) ||
      overlaps(len, lb, v, tb))
    return REL_E_ALIAS;
  const hipError_t e =
      rel::launch_cache_append(cache_P2, cache_V, len, p2, v, B, H, L_cap, d_h, dt == REL_BF16, stream);
  return e == hipSuccess ? REL_OK : REL_E_LAUNCH;
}

}  // extern "C"

rel_status relation_select_kernels(rel_kernel fwd, rel_kernel bwd) {
  auto ok = [](int k) { return k == REL_KERNEL_AUTO || k == REL_KERNEL_SCAN; };
  if (!ok(fwd) || !ok(bwd)) return REL_E_KERNEL;
  read_kernel_env();   // so that a later first use does not override this selection
  g_fwd_kernel.store(fwd, std::memory_order_relaxed);
  g_bwd_kernel.store(bwd, std::memory_order_relaxed);
  return REL_OK;
}

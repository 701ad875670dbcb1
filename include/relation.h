/*
 * relation.h - C ABI of librelation.so: the causal Self-Exchange Relation
 * forward (FlashRelation form), its backward, the model-side pre-steps
 * (RoPE, Givens head mixing), the Linear Relation forward and the Relation
 * Cache decode step on AMD Instinct MI355X (gfx950).
 *
 * Operator ("Ask Self, Ask Others: Relation Is All You Need", Eq. (1)-(3)),
 * per batch entry b and head h, for query row i (one-based) of T:
 *   U_ij = p1_i . p2_j / sqrt(d_h)
 *   R_ii = sigmoid(U_ii / tau_h)                  (Self)
 *   R_ij = SiLU(U_ij) - lambda * log(i),  j < i   (Exchange)
 *   R_ij = -inf,                          j > i
 *   Y_i  = sum_{j<=i} softmax(R_i)_j V_j
 * Execution follows the paper's factorised tiled scan (Sec. 5.1, Eq. (12)-(14)):
 * Exchange is scanned with running (max, sum, accumulator) and Self enters
 * once per row afterwards, so U, R and F are never materialised.
 * V is the information state after any head mixing (I~ in Eq. (4)-(5)); P1
 * and P2 are taken after any positional rotation. Heads are independent
 * (App. A.2.1).
 *
 * Common conventions
 *   - Tensors are device memory, contiguous row-major [B, H, T, d_h] (forward)
 *     or [B, H, d_h] / [B, H, L_cap, d_h] (decode); all of one dtype.
 *   - tau_s is HOST memory, float[H], read during the call (may be freed on
 *     return). Every tau must be finite and > 0 (the paper requires tau_S > 0).
 *   - lambda is the count-calibration coefficient; 0 gives the operator without
 *     count calibration.
 *   - The caller owns every buffer. The library allocates nothing and keeps
 *     no pointer after returning. Its global state: a per-device cache of the
 *     compute-unit count (written once, the same value by any caller); the
 *     kernel selection (relation_select_kernels, process-wide); and, for
 *     relation_decode_noalloc only, a fixed device array per GPU (loaded with
 *     the library's code object) and the cache of its per-device address.
 *   - All argument checks run on the host before any HIP call; on an error
 *     nothing is launched and no memory is touched.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *     caller synchronises. REL_E_LAUNCH reports a launch failure.
 *   - Tensor pointers must be 16-byte aligned, float arrays (LSE, dtau,
 *     dlambda) 4-byte aligned; an output range may not overlap any input
 *     range or another output range.
 *   - Supported: d_h in {32, 64, 128} for every entry point, and also 48 and
 *     80 (the paper's model geometries) for every entry point but
 *     relation_linear_fwd; 1 <= H <= REL_MAX_HEADS; B <= 65535.
 */
#ifndef RELATION_H
#define RELATION_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; the entry points
 * declared here are its only exports. */
#pragma GCC visibility push(default)

#define REL_MAX_HEADS 256

typedef enum {
  REL_OK = 0,
  REL_E_NULL = 1,      /* a required pointer is NULL                         */
  REL_E_SHAPE = 2,     /* B, H, T, d_h or L_cap out of range / overflow      */
  REL_E_DTYPE = 3,     /* unknown dtype                                      */
  REL_E_HEADDIM = 4,   /* d_h not supported                                  */
  REL_E_TAU = 5,       /* a tau is NaN, infinite or <= 0                     */
  REL_E_LAMBDA = 6,    /* lambda is NaN or infinite                          */
  REL_E_ALIGN = 7,     /* a pointer is misaligned (see conventions)          */
  REL_E_ALIAS = 8,     /* an output range overlaps an input or output range  */
  REL_E_WORKSPACE = 9, /* workspace missing or smaller than required         */
  REL_E_LAUNCH = 10,   /* a kernel launch failed                             */
  REL_E_PRESTEP = 11,  /* invalid rotary mode / base, pairing or Givens angle */
  REL_E_KERNEL = 12    /* unknown kernel selection                           */
} rel_status;

typedef enum { REL_F32 = 0, REL_BF16 = 1 } rel_dtype;

/* Rotary pair convention of the pre-step: pair k turns by pos * base^(-2k/d_h). */
typedef enum {
  REL_ROPE_NONE = 0,         /* no rotation                              */
  REL_ROPE_INTERLEAVED = 1,  /* pair k = (x_{2k}, x_{2k+1})              */
  REL_ROPE_HALF = 2          /* pair k = (x_k, x_{k + d_h/2})            */
} rel_rope;

/* Givens head pairings (App. A.2.3; one-based heads, H even). */
typedef enum {
  REL_PAIRS_A = 0,           /* (1,2), (3,4), ..., (H-1,H)               */
  REL_PAIRS_B = 1            /* (2,3), (4,5), ..., (H,1)                 */
} rel_pairing;

/*
 * relation_fwd - causal multi-head Relation forward without count
 * calibration (lambda = 0): the paper's Eq. (1)-(3) evaluated by the tiled
 * scan of Sec. 5.1. Equivalent to relation_fwd_ex(..., lambda = 0, ...).
 *
 *   P1, P2, V : in,  device [B, H, T, d_h], dtype dt
 *   tau_s     : in,  host float[H], per-head Self temperature
 *   Y         : out, device [B, H, T, d_h], dtype dt
 * Numerics: REL_BF16 computes both contractions on bf16 MFMA with fp32
 * accumulation, keeps the scan state and the Self term in fp32, rounds the
 * Exchange weights to bf16 as the second contraction's operand, and rounds Y
 * to bf16 (nearest-even). REL_F32 computes in fp32 throughout.
 */
rel_status relation_fwd(const void* P1, const void* P2, const void* V,
                        const float* tau_s, void* Y, int B, int H, int T,
                        int d_h, rel_dtype dt, hipStream_t stream);

/*
 * relation_fwd_ex - as relation_fwd, with the count calibration
 * -lambda * log(i) on every Exchange entry of row i (Eq. (2); i one-based).
 * lambda must be finite.
 */
rel_status relation_fwd_ex(const void* P1, const void* P2, const void* V,
                           const float* tau_s, float lambda, void* Y, int B,
                           int H, int T, int d_h, rel_dtype dt,
                           hipStream_t stream);

/*
 * relation_fwd_lse - the training forward: relation_fwd_ex plus the per-row
 * log normaliser the backward needs,
 *   LSE[b, h, i] = log( e^{S_i} + sum_{j<i} e^{SiLU(U_ij) - lambda log i} )
 *               = log sum_{j<=i} e^{R_ij}       (natural log, fp32)
 * i.e. log of the partition e^{S_i} + e^{A_i} of Eq. (6)-(7); row 1 gives S_1.
 *
 *   LSE : out, device float[B, H, T]
 * Y is identical to relation_fwd_ex's for the same arguments.
 */
rel_status relation_fwd_lse(const void* P1, const void* P2, const void* V,
                            const float* tau_s, float lambda, void* Y,
                            float* LSE, int B, int H, int T, int d_h,
                            rel_dtype dt, hipStream_t stream);

/*
 * relation_bwd_workspace_bytes - bytes of device workspace relation_bwd needs
 * for these sizes (per-row statistics and per-chunk scalar partials). 0 on
 * invalid sizes.
 */
size_t relation_bwd_workspace_bytes(int B, int H, int T, int d_h);

/*
 * relation_bwd_stored_workspace_bytes - bytes of device workspace with which
 * relation_bwd (dtype REL_BF16, d_h in {32, 48, 64, 80, 128}) stores dU once
 * instead of recomputing the evidence for dP1: the statistics and partials
 * of relation_bwd_workspace_bytes plus dU in bf16 for every strictly causal
 * (query, key) pair, in blocks of 32 queries x 16 keys (about B H T^2 bytes;
 * 2.1 GB for B = 1, H = 32, T = 8192). 0 on invalid sizes, or where that path
 * is not available (a head's dU blocks must stay below 2^31 bytes, i.e.
 * T <= 46,304).
 */
size_t relation_bwd_stored_workspace_bytes(int B, int H, int T, int d_h);

/*
 * relation_bwd - gradients of the forward (Eq. (1)-(3) with the count term of
 * Eq. (2)) for an upstream gradient dY = dL/dY:
 *   dP1, dP2, dV : dL/dP1, dL/dP2, dL/dV, device [B, H, T, d_h], dtype dt
 *   dtau         : dL/dtau_h summed over the batch, device float[H]
 *   dlambda      : dL/dlambda summed over batch and heads, device float[1]
 * The evidence is recomputed per tile from the saved row log normaliser (the
 * FlashRelation backward, App. A.3); with F = softmax(R) per row:
 *   dR_ij = F_ij (dY_i . V_j - dY_i . Y_i),
 *   dU_ij = dR_ij SiLU'(U_ij) (j < i),  dU_ii = dR_ii S_i (1 - S_i) / tau_h,
 *   dP1 = dU P2 / sqrt(d_h), dP2 = dU^T P1 / sqrt(d_h), dV = F^T dY,
 *   dtau_h = -sum_i dR_ii S_i (1 - S_i) U_ii / tau_h^2,
 *   dlambda = -sum_i log i sum_{j<i} dR_ij.
 *
 *   P1, P2, V, tau_s, lambda : the forward's inputs
 *   Y, LSE       : in, the forward's outputs from relation_fwd_lse with the
 *                  same inputs
 *   dY           : in, device [B, H, T, d_h], dtype dt
 *   workspace    : device scratch of >= relation_bwd_workspace_bytes bytes;
 *                  with >= relation_bwd_stored_workspace_bytes bytes (when
 *                  that is not 0) the bf16 MFMA path stores dU in it: the
 *                  key/value pass writes each dU block once and the query
 *                  pass forms dP1 = dU P2 from the stored blocks, instead of
 *                  recomputing U, dY V^T and the weights (same roundings: dU
 *                  is a bf16 MFMA operand on both paths)
 * Every output is overwritten (not accumulated into). The result is
 * deterministic: no atomics, scalar sums in a fixed order (fp64 across rows
 * chunks, heads and batch).
 * Numerics: REL_BF16 with d_h in {32, 48, 64, 80, 128} recomputes both evidence
 * products on bf16 MFMA and rounds F and dU to bf16 as operands of the
 * gradient products (fp32 accumulation); other cases compute in fp32
 * throughout.
 */
rel_status relation_bwd(const void* P1, const void* P2, const void* V,
                        const float* tau_s, float lambda, const void* Y,
                        const float* LSE, const void* dY, void* dP1, void* dP2,
                        void* dV, float* dtau, float* dlambda, int B, int H,
                        int T, int d_h, rel_dtype dt, void* workspace,
                        size_t ws_bytes, hipStream_t stream);

/*
 * relation_prestep - the model-side steps before the operator, in one pass
 * over HBM:
 *   - full-head rotary position encoding of P1 and P2 (the paper's models use
 *     base 10^4, App. B.3): rotary pair k of the row at zero-based position
 *     pos = pos0[b] + t turns by pos * rope_base^(-2k/d_h),
 *       (x_a, x_b) -> (x_a cos - x_b sin, x_a sin + x_b cos);
 *   - Givens mixing of the information heads (Eq. (4), App. A.2.2): for the
 *     k-th pair (a, b) of `pairing`, with angle theta[k],
 *       I~(a) = cos I(a) - sin I(b),   I~(b) = sin I(a) + cos I(b),
 *     applied to all d_h channels of every row.
 *
 *   P1, P2, I     : in, device [B, H, T, d_h], dtype dt
 *   pos0          : in, device int32[B] (position of row 0 per sequence; a
 *                   decode token uses pos0 = its cache length), or NULL for 0
 *   rope          : rotary convention; REL_ROPE_NONE copies P1 / P2
 *   rope_base     : finite, > 1 (ignored for REL_ROPE_NONE)
 *   theta         : HOST float[H/2], the pairing's angles in pair order (H
 *                   must be even), or NULL for no mixing (I is copied)
 *   P1o, P2o, Io  : out, device [B, H, T, d_h]; each may be exactly its own
 *                   input (in place) and may overlap nothing else
 * Numerics: fp32 arithmetic; the rotary angle is formed and range-reduced in
 * fp64 before an fp32 sincos; bf16 outputs are rounded to nearest even.
 */
rel_status relation_prestep(const void* P1, const void* P2, const void* I,
                            const int32_t* pos0, rel_rope rope,
                            float rope_base, const float* theta,
                            rel_pairing pairing, void* P1o, void* P2o,
                            void* Io, int B, int H, int T, int d_h,
                            rel_dtype dt, hipStream_t stream);

/*
 * relation_fwd_model_workspace_bytes - device workspace relation_fwd_model
 * needs (the three pre-stepped tensors). 0 on invalid sizes or dtype.
 */
size_t relation_fwd_model_workspace_bytes(int B, int H, int T, int d_h,
                                          rel_dtype dt);

/*
 * relation_fwd_model - the operator on raw projections, as the paper's model
 * computes it: relation_prestep into the workspace, then relation_fwd_lse
 * (LSE may be NULL) on the rotated P1 / P2 and the mixed information I~.
 * Arguments as for those two calls; Y and LSE may not overlap the inputs or
 * the workspace. The workspace has three 256-byte aligned slots (rotated P1,
 * rotated P2, mixed I, in that order); after the call the last two hold the
 * pre-stepped P2 and I. Where the bf16 MFMA forward rotates P1 itself as it
 * loads each query tile (REL_BF16, d_h in {32, 48, 64, 80, 128}, interleaved
 * pairs, or half-split pairs with d_h a multiple of 32) the first slot is
 * not written, and the result equals pre-step then forward bit for bit;
 * otherwise the first slot holds the rotated P1. A backward on the rotated
 * coordinates takes rotated P1 from relation_prestep.
 */
rel_status relation_fwd_model(const void* P1, const void* P2, const void* I,
                              const int32_t* pos0, rel_rope rope,
                              float rope_base, const float* theta,
                              rel_pairing pairing, const float* tau_s,
                              float lambda, void* Y, float* LSE, int B, int H,
                              int T, int d_h, rel_dtype dt, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

/*
 * relation_linear_workspace_bytes - device workspace relation_linear_fwd
 * needs (at most one d_h x d_h fp32 state and d_h decays per 64-token chunk
 * and head, and two fp32 row factors per token and head). 0 on invalid
 * sizes.
 */
size_t relation_linear_workspace_bytes(int B, int H, int T, int d_h);

/*
 * relation_linear_fwd - the Linear Relation forward (Sec. 5.2, Eq. (15)-(17),
 * App. A.4): per head, with C_0 = 0 (d_h x d_h),
 *   S_t = sigmoid(p1_t . p2_t / (tau_h sqrt(d_h))),
 *   q_t = p1_t / |p1_t|,  k_t = p2_t / |p2_t|   (0 for a zero row),
 *   C-_t = Diag(alpha_t) C_{t-1},  Y_t = I_t + S_t (C-_t)^T q_t,
 *   C_t = C-_t + S_t k_t I_t^T        (read before write).
 * Evaluated in 64-token chunks taken in groups of consecutive chunks (up to
 * 16, chosen from the sizes and the device's compute-unit count; one for fp32
 * inputs): per-group state contributions, a scan over groups, then each
 * chunk's outputs from its entering state, stepped from chunk to chunk
 * within a group. The group size changes only the summation order.
 *
 *   P1, P2, I : in, device [B, H, T, d_h], dtype dt (P1 / P2 after RoPE, I the
 *               mixed information state)
 *   alpha     : in, device fp32 [B, H, T, d_h], the channel-wise retention in
 *               (0, 1]; values outside are clamped to [1e-30, 1] (NaN -> 1e-30)
 *   tau_s     : host float[H]
 *   Y         : out, device [B, H, T, d_h], dtype dt
 *   state_out : out, device fp32 [B, H, d_h, d_h] = C_T (rows: relation
 *               coordinate, columns: information channel), or NULL
 *   workspace : device scratch of >= relation_linear_workspace_bytes
 * Numerics: fp32 arithmetic throughout; bf16 Y rounded to nearest even.
 */
rel_status relation_linear_fwd(const void* P1, const void* P2, const void* I,
                               const float* alpha, const float* tau_s,
                               void* Y, float* state_out, int B, int H, int T,
                               int d_h, rel_dtype dt, void* workspace,
                               size_t ws_bytes, hipStream_t stream);

/*
 * relation_decode_workspace_bytes - bytes of device workspace relation_decode
 * needs for these sizes (split-history partial states). 0 on invalid sizes.
 */
size_t relation_decode_workspace_bytes(int B, int H, int L_cap, int d_h);

/*
 * relation_decode - one autoregressive step against a Relation Cache
 * (Eq. (18), App. A.5): the cache holds the historical P2 rows and
 * information rows of each sequence; the new token's p1 is matched against
 * them, its own p1 . p2 gives the Self entry, and the output is row L_b + 1 of
 * the forward on [cache rows 0..L_b-1; new token].
 *
 *   p1, p2, v          : in, device [B, H, d_h], the new token's states
 *   cache_P2, cache_V  : in, device [B, H, L_cap, d_h]; rows >= len[b] are
 *                        never read (they may hold anything, NaN included)
 *   len                : in, device int32[B], cached rows per sequence; a value
 *                        outside [0, L_cap] is clamped into that range
 *   tau_s, lambda      : as for relation_fwd_ex (new token position L_b + 1)
 *   y                  : out, device [B, H, d_h]
 *   workspace          : device scratch of >= relation_decode_workspace_bytes
 * The cache is not modified; append with relation_cache_append afterwards.
 */
rel_status relation_decode(const void* p1, const void* p2, const void* v,
                           const void* cache_P2, const void* cache_V,
                           const int32_t* len, const float* tau_s,
                           float lambda, void* y, int B, int H, int L_cap,
                           int d_h, rel_dtype dt, void* workspace,
                           size_t ws_bytes, hipStream_t stream);

/*
 * relation_decode_noalloc - relation_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same arguments without a workspace, the same
 * kernels and the same result. The partial states live in a device array of
 * the library, REL_DECODE_SCRATCH_BYTES (32 MiB) per GPU, held by each GPU the
 * library runs on until the process ends; the call allocates and frees
 * nothing. REL_E_WORKSPACE when relation_decode_workspace_bytes(B, H, L_cap,
 * d_h) exceeds that size (then nothing is launched), REL_E_LAUNCH if the
 * array's address cannot be found. Every call on one GPU uses the same array
 * (each call writes every state it reads, so nothing carries over): calls
 * that may run at the same time on one GPU (other streams, other threads)
 * race and must be serialised by the caller.
 */
#define REL_DECODE_SCRATCH_BYTES (32u << 20)
rel_status relation_decode_noalloc(const void* p1, const void* p2, const void* v,
                                   const void* cache_P2, const void* cache_V,
                                   const int32_t* len, const float* tau_s,
                                   float lambda, void* y, int B, int H,
                                   int L_cap, int d_h, rel_dtype dt,
                                   hipStream_t stream);

/*
 * relation_cache_append - the cache update of App. A.5.3: write the token's
 * p2 and v ([B, H, d_h]) as row len[b] of cache_P2 / cache_V and increment
 * len[b]. A sequence whose len[b] is already >= L_cap (or < 0) is left
 * unchanged, len included.
 */
rel_status relation_cache_append(void* cache_P2, void* cache_V, int32_t* len,
                                 const void* p2, const void* v, int B, int H,
                                 int L_cap, int d_h, rel_dtype dt,
                                 hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* relation_status_str(rel_status s);

/* Kernel family of the bf16 forward and backward. */
typedef enum {
  REL_KERNEL_AUTO = 0,  /* the MFMA kernels wherever they apply (default)  */
  REL_KERNEL_SCAN = 1   /* the row-scan kernels (to run and test them alone) */
} rel_kernel;

/*
 * relation_select_kernels - which kernels the bf16 forward family
 * (relation_fwd, relation_fwd_ex, relation_fwd_lse, relation_fwd_model) and
 * relation_bwd run. The selection is process-wide; calls made after this
 * one returns use it. Before any call to it, the selection comes from the
 * environment variables RELATION_FWD_KERNEL and RELATION_BWD_KERNEL (the
 * value "scan" selects REL_KERNEL_SCAN), read once, the first time a
 * selection is needed. No HIP call; REL_E_KERNEL for a value outside
 * rel_kernel (and then nothing changes).
 */
rel_status relation_select_kernels(rel_kernel fwd, rel_kernel bwd);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* RELATION_H */

"""Plain fp64 CPU oracle for the causal Self-Exchange Relation (SER / MHR).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: only the test suite, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP kernels and is deliberately slow and
literal: it materialises the T x T relation matrix R and the flow F per head.

Source: "Ask Self, Ask Others: Relation Is All You Need" (arXiv 2608.20172),
abbreviated [paper] below, and the author's blog post on the derivation
(qingkeai.online, "Attention -> Relation"), abbreviated [blog].

Definition followed by ``relation_head`` (one head, rows of P1/P2/V are tokens):
  U_ij = p1_i . p2_j / sqrt(d_h)                        [paper] Eq. (1)
  S_i  = sigmoid(U_ii / tau_S)                          [paper] Eq. (2)
  E_ij = SiLU(U_ij) = U_ij * sigmoid(U_ij)              [paper] Eq. (2)
  R_ii = S_i;  R_ij = E_ij - lambda * log(i) for j < i;  R_ij = -inf for j > i
        with i one-based                                [paper] Eq. (2), App. A intro
  F_i  = softmax(R_i);  Y_i = sum_{j<=i} F_ij V_j       [paper] Eq. (3)
V stands for the information state after head mixing (I~ in [paper] Eq. (4)-(5));
head mixing and RoPE happen before this operator and are not part of it.

Readings taken where the pages leave a choice open:
  * lambda (the count calibration) is an argument, default 0 (the paper's
    "no count calibration" variant, Table 3); tau_S is one value per head.
  * S_i enters R as a logit (it is exponentiated by the softmax), not rescaled.
  * Decode: the new token sits at one-based position L+1 after L cached rows;
    its row is the definition's last row on [cache rows; new token]
    ([paper] Eq. (18), App. A.5).

Gradients (``relation_head_bwd`` / ``relation_bwd``): the derivatives of
sum(Y * dY) with respect to P1, P2, V, tau_S and lambda, by the chain rule
through the same three equations (the pages give no backward pass; this is
plain calculus on the definition, written out on the materialised matrices):
  dV = F^T dY;  dF_ij = dY_i . V_j;  D_i = dY_i . Y_i;  dR = F * (dF - D)
  dU_ii = dR_ii S_i (1 - S_i) / tau;   dU_ij = dR_ij SiLU'(U_ij)  (j < i)
  dP1 = dU P2 / sqrt(d_h);  dP2 = dU^T P1 / sqrt(d_h)
  dtau = -sum_i dR_ii S_i (1 - S_i) U_ii / tau^2;  dlambda = -sum_{j<i} dR_ij log i
with SiLU'(u) = sigmoid(u) (1 + u (1 - sigmoid(u))). ``row_lse`` gives the
per-row log normaliser LSE_i = log sum_{j<=i} exp(R_ij) that a training
forward hands to its backward.

Cross-check routes (exact algebra per the paper; used only to pin this file):
  * ``factorized_head``: Eq. (6)-(9) / App. A.1.2-A.1.6.
  * ``flash_scan_head``: the tiled (m, l, z) Exchange scan, Eq. (12)-(14) /
    App. A.3, with caller-chosen tile boundaries.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "sigmoid", "silu", "silu_grad", "evidence", "relation_matrix", "flow", "relation_head",
    "relation_fwd", "relation_rows", "relation_decode", "row_lse", "relation_head_bwd",
    "relation_bwd", "relation_head_bwd_sampled", "factorized_head", "flash_scan_head",
]


def sigmoid(x):
    """Logistic function, evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(x):
    """SiLU(x) = x * sigmoid(x): the Exchange map ([paper] Eq. (2))."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def silu_grad(x):
    """d SiLU(x) / dx = sigmoid(x) (1 + x (1 - sigmoid(x)))."""
    x = np.asarray(x, dtype=np.float64)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def evidence(p1, p2):
    """U = P1 P2^T / sqrt(d_h) for one head ([paper] Eq. (1))."""
    d_h = p1.shape[-1]
    return (p1 @ p2.T) / math.sqrt(d_h)


def relation_matrix(p1, p2, tau, lam=0.0):
    """The causal relation matrix R of one head ([paper] Eq. (2)).

    p1, p2: float64 [T, d_h]. Returns float64 [T, T] with -inf above the diagonal.
    """
    T = p1.shape[0]
    U = evidence(p1, p2)
    R = np.full((T, T), -np.inf)
    below = np.tril(np.ones((T, T), dtype=bool), k=-1)
    i_one_based = np.arange(1, T + 1, dtype=np.float64)
    count = lam * np.log(i_one_based)                  # -lambda log i, row-wise
    E = silu(U)
    R[below] = (E - count[:, None])[below]
    diag = np.arange(T)
    R[diag, diag] = sigmoid(U[diag, diag] / float(tau))
    return R


def flow(R):
    """Row-wise softmax of R ([paper] Eq. (3)); exp(-inf) contributes 0."""
    mx = np.max(R, axis=1, keepdims=True)
    W = np.exp(R - mx)
    return W / np.sum(W, axis=1, keepdims=True)


def relation_head(p1, p2, v, tau, lam=0.0, return_flow=False):
    """Y = F V for one head; all arguments float64 [T, d_h]."""
    F = flow(relation_matrix(p1, p2, tau, lam))
    Y = F @ v
    return (Y, F) if return_flow else Y


def relation_fwd(P1, P2, V, tau, lam=0.0):
    """Multi-head forward: [B, H, T, d_h] float64 arrays, tau float[H].

    Heads are independent ([paper] Sec. 3.2, App. A.2.1): loop over (b, h).
    """
    B, H, T, _ = P1.shape
    Y = np.empty(V.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            Y[b, h] = relation_head(P1[b, h], P2[b, h], V[b, h], tau[h], lam)
    return Y


def relation_rows(p1, p2, v, tau, lam, rows):
    """Selected output rows of one head, each straight from the definition.

    rows: zero-based row indices r; row r is token i = r + 1. Row r reads only
    p1[r], p2[:r+1] and v[:r+1], so large T costs O(r d_h) per row.
    """
    d_h = p1.shape[-1]
    out = np.empty((len(rows), v.shape[1]), dtype=np.float64)
    for k, r in enumerate(rows):
        u = (p2[: r + 1] @ p1[r]) / math.sqrt(d_h)        # U_{i, 1..i}
        logits = silu(u) - lam * math.log(r + 1)           # Exchange entries
        logits[r] = sigmoid(np.array([u[r] / float(tau)]))[0]  # Self entry
        w = np.exp(logits - logits.max())
        out[k] = (w / w.sum()) @ v[: r + 1]
    return out


def relation_decode(p1, p2, v, cache_P2, cache_V, lens, tau, lam=0.0):
    """One decode step against a Relation Cache ([paper] Eq. (18), App. A.5).

    p1, p2, v: [B, H, d_h]; cache_P2, cache_V: [B, H, L_cap, d_h]; lens: [B].
    The output for (b, h) is the last row of the forward on the sequence
    [cache rows 0..L_b-1; new token]. Cache rows at or past L_b are not read.
    """
    B, H, d_h = p1.shape
    y = np.empty((B, H, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            P2seq = np.concatenate([cache_P2[b, h, :L], p2[b, h][None]], axis=0)
            Vseq = np.concatenate([cache_V[b, h, :L], v[b, h][None]], axis=0)
            P1row = np.zeros_like(P2seq)
            P1row[L] = p1[b, h]
            y[b, h] = relation_rows(P1row, P2seq, Vseq, tau[h], lam, [L])[0]
    return y


def row_lse(p1, p2, tau, lam=0.0):
    """LSE_i = log sum_{j<=i} exp(R_ij) per row of one head (natural log)."""
    R = relation_matrix(p1, p2, tau, lam)
    mx = np.max(R, axis=1)
    return mx + np.log(np.sum(np.exp(R - mx[:, None]), axis=1))


def relation_head_bwd(p1, p2, v, tau, lam, dy, return_terms=False):
    """Gradients of sum(Y * dy) for one head: (dP1, dP2, dV, dtau, dlambda).

    Chain rule through [paper] Eq. (1)-(3) on the materialised U, R, F.
    With return_terms, also a dict of per-row quantities behind the two
    scalars: tau_terms (row i's share of dtau), lam_terms (row i's share of
    dlambda), F_self (F_ii), U_self (U_ii), S (S_i), dR_self (dR_ii).
    """
    T, d_h = p1.shape
    tau = float(tau)
    U = evidence(p1, p2)
    F = flow(relation_matrix(p1, p2, tau, lam))
    Y = F @ v
    dV = F.T @ dy                                    # Y = F V
    dF = dy @ v.T
    D = np.sum(dy * Y, axis=1)                       # sum_j F_ij dF_ij
    dR = F * (dF - D[:, None])                       # softmax backward; 0 above the diagonal
    below = np.tril(np.ones((T, T), dtype=bool), k=-1)
    diag = np.arange(T)
    dU = np.zeros((T, T))
    dU[below] = (dR * silu_grad(U))[below]           # Exchange: R_ij = SiLU(U_ij) - lambda log i
    s = sigmoid(U[diag, diag] / tau)                 # Self: R_ii = sigmoid(U_ii / tau)
    dU[diag, diag] = dR[diag, diag] * s * (1.0 - s) / tau
    dP1 = dU @ p2 / math.sqrt(d_h)                   # U = P1 P2^T / sqrt(d_h)
    dP2 = dU.T @ p1 / math.sqrt(d_h)
    dtau = float(np.sum(dR[diag, diag] * s * (1.0 - s) * (-U[diag, diag] / tau ** 2)))
    log_i = np.log(np.arange(1, T + 1, dtype=np.float64))
    dlam = float(-np.sum(np.where(below, dR, 0.0) * log_i[:, None]))
    if return_terms:
        terms = dict(tau_terms=dR[diag, diag] * s * (1.0 - s) * (-U[diag, diag] / tau ** 2),
                     lam_terms=-log_i * np.sum(np.where(below, dR, 0.0), axis=1),
                     F_self=F[diag, diag].copy(), U_self=U[diag, diag].copy(), S=s,
                     dR_self=dR[diag, diag].copy())
        return dP1, dP2, dV, dtau, dlam, terms
    return dP1, dP2, dV, dtau, dlam


def relation_bwd(P1, P2, V, tau, lam, dY):
    """Multi-head gradients: dP1, dP2, dV [B, H, T, d_h], dtau [H] (tau is
    shared across the batch), dlambda (scalar, shared by every head)."""
    B, H, T, _ = P1.shape
    dP1 = np.empty(P1.shape)
    dP2 = np.empty(P2.shape)
    dV = np.empty(V.shape)
    dtau = np.zeros(H)
    dlam = 0.0
    for b in range(B):
        for h in range(H):
            g = relation_head_bwd(P1[b, h], P2[b, h], V[b, h], tau[h], lam, dY[b, h])
            dP1[b, h], dP2[b, h], dV[b, h] = g[0], g[1], g[2]
            dtau[h] += g[3]
            dlam += g[4]
    return dP1, dP2, dV, dtau, dlam


def relation_head_bwd_sampled(p1, p2, v, tau, lam, dy, rows, cols, block=256):
    """Selected gradient entries of one head without the T x T matrices, for
    sizes where ``relation_head_bwd`` does not fit: dP1 at query rows `rows`,
    dV and dP2 at key rows `cols`, and the head's dtau. The same chain rule
    as ``relation_head_bwd``, evaluated row by row (dP1_i needs row i of R, F,
    dF) and column by column (dV_j, dP2_j need column j), after one
    block-by-block pass of the forward for every row's LSE_i, Y_i and D_i."""
    p1, p2, v, dy = (np.asarray(x, dtype=np.float64) for x in (p1, p2, v, dy))
    T, d_h = p1.shape
    tau = float(tau)
    c = 1.0 / math.sqrt(d_h)
    log_i = np.log(np.arange(1, T + 1, dtype=np.float64))
    diag_u = np.sum(p1 * p2, axis=1) * c
    S = sigmoid(diag_u / tau)
    lse = np.empty(T)
    Y = np.empty((T, d_h))
    for r0 in range(0, T, block):                     # forward, `block` query rows at a time
        r1 = min(T, r0 + block)
        U = (p1[r0:r1] @ p2.T) * c
        R = silu(U) - lam * log_i[r0:r1, None]
        i = np.arange(r0, r1)[:, None]
        j = np.arange(T)[None, :]
        R = np.where(j < i, R, -np.inf)
        R[np.arange(r1 - r0), np.arange(r0, r1)] = S[r0:r1]
        mx = np.max(R, axis=1, keepdims=True)
        W = np.exp(R - mx)
        lse[r0:r1] = mx[:, 0] + np.log(np.sum(W, axis=1))
        Y[r0:r1] = (W / np.sum(W, axis=1, keepdims=True)) @ v
    D = np.sum(dy * Y, axis=1)
    dP1 = np.empty((len(rows), d_h))
    for n, i in enumerate(rows):                      # row i: F_i., dF_i. over keys j <= i
        u = (p2[: i + 1] @ p1[i]) * c
        R = silu(u) - lam * log_i[i]
        R[i] = S[i]
        F = np.exp(R - lse[i])
        dR = F * (v[: i + 1] @ dy[i] - D[i])
        dU = dR * silu_grad(u)
        dU[i] = dR[i] * S[i] * (1.0 - S[i]) / tau
        dP1[n] = (dU @ p2[: i + 1]) * c
    dV = np.empty((len(cols), d_h))
    dP2 = np.empty((len(cols), d_h))
    for n, j in enumerate(cols):                      # column j: F_.j, dF_.j over queries i >= j
        u = (p1[j:] @ p2[j]) * c
        R = silu(u) - lam * log_i[j:]
        R[0] = S[j]
        F = np.exp(R - lse[j:])
        dR = F * (dy[j:] @ v[j] - D[j:])
        dU = dR * silu_grad(u)
        dU[0] = dR[0] * S[j] * (1.0 - S[j]) / tau
        dV[n] = F @ dy[j:]
        dP2[n] = (dU @ p1[j:]) * c
    F_self = np.exp(S - lse)
    dR_self = F_self * (np.sum(dy * v, axis=1) - D)
    dtau = float(np.sum(dR_self * S * (1.0 - S) * (-diag_u / tau ** 2)))
    return dict(dP1=dP1, dV=dV, dP2=dP2, dtau=dtau, lse=lse, Y=Y, F_self=F_self, S=S, U_self=diag_u)


def relation_head_dp1_rows(p1, p2, v, tau, lam, dy, rows):
    """dP1 at query rows `rows` of one head, each row on its own: row i's
    relation logits, flow F_i, output Y_i and D_i = dY_i . Y_i need only
    p1[i], p2[:i+1], v[:i+1] and dy[i], so each row costs O(i d_h) at any T.
    The chain rule is the one of ``relation_head_bwd`` restricted to row i:
    dR_ij = F_ij (dY_i . V_j - D_i), dU_ij = dR_ij SiLU'(U_ij) below the
    diagonal and dR_ii S_i (1 - S_i) / tau on it, dP1_i = sum_j dU_ij p2_j / sqrt(d_h)."""
    p1, p2, v, dy = (np.asarray(x, dtype=np.float64) for x in (p1, p2, v, dy))
    d_h = p1.shape[-1]
    c = 1.0 / math.sqrt(d_h)
    tau = float(tau)
    out = np.empty((len(rows), d_h))
    for n, i in enumerate(rows):
        u = (p2[: i + 1] @ p1[i]) * c
        s = sigmoid(np.array([u[i] / tau]))[0]
        R = silu(u) - lam * math.log(i + 1)
        R[i] = s
        W = np.exp(R - R.max())
        F = W / W.sum()
        y = F @ v[: i + 1]
        dR = F * (v[: i + 1] @ dy[i] - float(dy[i] @ y))
        dU = dR * silu_grad(u)
        dU[i] = dR[i] * s * (1.0 - s) / tau
        out[n] = (dU @ p2[: i + 1]) * c
    return out


# ---------------------------------------------------------------------------
# Cross-check routes (pins for the definition above; never used by the kernels)
# ---------------------------------------------------------------------------

def _lse(a):
    """log sum exp over a 1-D array; -inf for an empty array ([paper] App. A.1.7)."""
    if a.size == 0:
        return -np.inf
    m = np.max(a)
    return m + math.log(np.sum(np.exp(a - m)))


def factorized_head(p1, p2, v, tau, lam=0.0):
    """Self mass / Exchange mass / Exchange allocation route, Eq. (6)-(9).

    Returns dict with Y, S, A, F_self (= F_ii), g, pi (strictly lower, rows sum
    to 1 for i > 1) and Ibar (the normalised historical summary, NaN on row 1).
    """
    T = p1.shape[0]
    U = evidence(p1, p2)
    d = np.arange(T)
    S = sigmoid(U[d, d] / float(tau))
    E = silu(U)
    A = np.empty(T)
    pi = np.zeros((T, T))
    Ibar = np.full(v.shape, np.nan)
    for r in range(T):
        i = r + 1
        LE = _lse(E[r, :r])                          # Eq. (6)
        A[r] = LE - lam * math.log(i)
        if r > 0:
            w = np.exp(E[r, :r] - np.max(E[r, :r]))
            pi[r, :r] = w / w.sum()                  # Eq. (8)
            Ibar[r] = pi[r, :r] @ v[:r]
    F_self = sigmoid(S - A)                          # Eq. (7)
    g = sigmoid(A - S)
    Y = F_self[:, None] * v                          # Eq. (9)
    Y[1:] += g[1:, None] * Ibar[1:]
    return dict(Y=Y, S=S, A=A, F_self=F_self, g=g, pi=pi, Ibar=Ibar)


def flash_scan_head(p1, p2, v, tau, lam=0.0, bounds=None):
    """Tiled historical Exchange scan, Eq. (12)-(14) / App. A.3.

    bounds: increasing key-tile boundaries starting at 0 (e.g. [0, 3, 7, ...]);
    default one tile per key. Self is not part of the scan; it enters once,
    after the scan, through A_i and g_i. Row 1 follows App. A.1.7 (Y_1 = V_1).
    """
    T, d_h = p1.shape
    if bounds is None:
        bounds = list(range(T + 1))
    bounds = list(bounds)
    if bounds[-1] < T:
        bounds.append(T)
    Y = np.empty(v.shape, dtype=np.float64)
    for r in range(T):
        i = r + 1
        m, l, z = -np.inf, 0.0, np.zeros(v.shape[1])    # empty-set state
        for t0, t1 in zip(bounds[:-1], bounds[1:]):
            t1 = min(t1, r)                              # historical j < i only
            if t0 >= t1:
                break
            u = (p2[t0:t1] @ p1[r]) / math.sqrt(d_h)
            E = silu(u)
            m_new = max(m, float(np.max(E)))
            scale = math.exp(m - m_new) if m != -np.inf else 0.0
            p = np.exp(E - m_new)
            l = scale * l + float(np.sum(p))
            z = scale * z + p @ v[t0:t1]
            m = m_new
        S = float(sigmoid(np.array([(p1[r] @ p2[r]) / math.sqrt(d_h) / float(tau)]))[0])
        if r == 0:
            Y[r] = v[r]                                  # A_1 = -inf: g_1 = 0
            continue
        A = m + math.log(l) - lam * math.log(i)          # Eq. (13)-(14)
        g = float(sigmoid(np.array([A - S]))[0])
        Y[r] = (1.0 - g) * v[r] + g * (z / l)
    return Y

"""First-order rounding-error bars for an fp32 evaluation of the operator and
of its gradients, used where the fixed fp32 bar (per-row normwise 1e-5) does
not apply: inputs whose evidence U reaches 30-45, where every fp32 rounding of
U moves a weight by a relative amount proportional to |U|.

Error model (u = 2^-24, the fp32 unit roundoff):
  - each fp32 +, -, *, / rounds with relative error <= u; exp, log and the
    reciprocal are within 1 ulp, i.e. <= 2u relative;
  - a sum of n products or terms accumulated in fp32, in any order of depth
    <= n, is within LAM * sqrt(n) * u * (the same sum of absolute values):
    the probabilistic bound of Higham & Mary ("A New Approach to
    Probabilistic Rounding Error Analysis", SIAM J. Sci. Comput. 41(5),
    2019), which holds with probability >= 1 - 2n exp(-LAM^2 / 2) per sum
    when the rounding errors are independent and of mean zero; LAM = 6.
Errors are propagated to first order (second-order terms are below u^2 |U|^2
d ~ 1e-8 relative here). Every quantity the bars are built from is the fp64
oracle's ([paper] Eq. (1)-(3)); the bars are elementwise and absolute.

Forward, per row i (one-based position i), natural-log units. With
k = 1/sqrt(d_h) and A_ij = k sum_c |p1_ic p2_jc|:
  dU_ij   <= u (LAM sqrt(d_h) A_ij + 2 |U_ij|)           dot product, scale
  eps_ij  <= 1.1 dU_ij + u (8 |E_ij| + 2 |m_i| + 2 lam log i + 4)
             for an Exchange weight e^(E_ij - lam log i - m_i)
             (|SiLU'| <= 1.1; SiLU and the shift by the running maximum m_i
             round on quantities of size |E| and |m|; the exponential's ulp)
  eps_ii  <= 0.25 (dU_ii + 2u |U_ii|) / tau + 6u      Self: sigmoid(U_ii/tau)
  alpha_i  = LAM sqrt(2 i) u + 2u                      accumulation of O and l
             over i terms plus up to i rescalings
  |dY_ic| <= sum_j F_ij eps_ij |V_jc - Y_ic|
             + alpha_i (sum_j F_ij |V_jc| + |Y_ic|) + 3u |Y_ic|
(a relative error eps_j on weight j moves Y_i by F_ij eps_j (V_j - Y_i)).

Backward (the chain of relation_head_bwd, each factor carrying its error):
  LSE_i:  dLSE_i <= sum_j F_ij eps_ij + alpha_i + u |LSE_i|
  F_ij recomputed from U and the stored LSE: phi_ij = eps_ij + dLSE_i
  D_i = dY_i . Y_i (stored Y): the weight errors move Y_i by
     sum_j F_ij eps_ij (V_j - Y_i), hence D_i by sum_j eps_ij dR_ij, so
     dD_i <= sum_j eps_ij |dR_ij| + alpha_i sum_c |dY_ic| (sum_j F_ij |V_jc|
             + |Y_ic|) + (LAM sqrt(d_h) + 3) u sum_c |dY_ic Y_ic|
  dF_ij = dY_i . V_j: eta_ij = LAM sqrt(d_h) u sum_c |dY_ic V_jc|
  dR_ij = F_ij (dF_ij - D_i):
     ddR_ij <= phi_ij |dR_ij| + F_ij (eta_ij + dD_i) + 2u |dR_ij|
  g_ij = SiLU'(U_ij) (j < i; |SiLU''| <= 1/2) or S_i (1 - S_i) / tau (j = i;
     |d/dU| <= 0.1 / tau^2): dg_ij <= |g'| dU_ij + 6u |g_ij|
  dU_ij = dR_ij g_ij: ddU_ij <= ddR_ij |g_ij| + |dR_ij| dg_ij + u |dU_ij|
  dV_j  = sum_i F_ij dY_i:
     |d dV_jc| <= sum_i F_ij (phi_ij + beta) |dY_ic|,  beta = LAM sqrt(T) u
  dP1_i = k sum_j dU_ij p2_j:
     |d dP1_ic| <= k sum_j (ddU_ij + (beta + 2u) |dU_ij|) |p2_jc|
  dP2_j = k sum_i dU_ij p1_i: the same with the roles of i and j swapped;
  dtau = sum_i dR_ii q_i, q_i = -S_i (1 - S_i) U_ii / tau^2
     (|dq_i/dU_ii| <= (0.1 |U_ii| + 0.25) / tau^2):
     |d dtau| <= sum_i (ddR_ii |q_i| + |dR_ii| (|dq/dU| dU_ii + 6u |q_i|))
                 + beta sum_i |dR_ii q_i|
  dlambda = sum_i log i dR_ii:
     |d dlambda| <= sum_i log i (ddR_ii + (beta + 2u) |dR_ii|).
"""
import math

import numpy as np

from oracle import relation_oracle as O

U_RND = 2.0 ** -24
LAM = 6.0


def _head_terms(p1, p2, tau, lam):
    """fp64 U, A, E, m, F and the per-weight log error bound eps of one head."""
    T, d = p1.shape
    k = 1.0 / math.sqrt(d)
    U = O.evidence(p1, p2)
    A = (np.abs(p1) @ np.abs(p2).T) * k
    dU = U_RND * (LAM * math.sqrt(d) * A + 2.0 * np.abs(U))
    R = O.relation_matrix(p1, p2, tau, lam)
    F = O.flow(R)
    E = O.silu(U)
    below = np.tril(np.ones((T, T), dtype=bool), k=-1)
    m = np.array([np.max(E[i, :i]) if i > 0 else 0.0 for i in range(T)])
    logi = np.log(np.arange(1, T + 1, dtype=np.float64))
    eps = 1.1 * dU + U_RND * (8.0 * np.abs(E) + 2.0 * np.abs(m)[:, None]
                              + 2.0 * abs(lam) * logi[:, None] + 4.0)
    diag = np.arange(T)
    eps[diag, diag] = 0.25 * (dU[diag, diag] + 2.0 * U_RND * np.abs(U[diag, diag])) / tau + 6.0 * U_RND
    eps = np.where(below | (np.arange(T)[:, None] == np.arange(T)[None, :]), eps, 0.0)
    alpha = LAM * np.sqrt(2.0 * np.arange(1, T + 1)) * U_RND + 2.0 * U_RND
    return dict(U=U, dU=dU, F=F, eps=eps, alpha=alpha, R=R, below=below, logi=logi)


def fwd_head_bar(p1, p2, v, tau, lam=0.0, terms=None):
    """Elementwise bound |Y_fp32 - Y| [T, d_h] for one head (fp64 inputs)."""
    t = terms or _head_terms(p1, p2, tau, lam)
    F, eps, alpha = t["F"], t["eps"], t["alpha"]
    Y = F @ v
    Fe = F * eps
    # sum_j F_ij eps_ij |V_jc - Y_ic|, summed row by row (T x T x d_h stays small)
    spread = np.empty_like(Y)
    for i in range(Y.shape[0]):
        spread[i] = Fe[i] @ np.abs(v - Y[i])
    return spread + alpha[:, None] * (F @ np.abs(v) + np.abs(Y)) + 3.0 * U_RND * np.abs(Y)


def fwd_bar(P1, P2, V, tau, lam=0.0):
    """fwd_head_bar over [B, H, T, d_h] (fp64)."""
    out = np.empty(V.shape)
    for b in range(P1.shape[0]):
        for h in range(P1.shape[1]):
            out[b, h] = fwd_head_bar(P1[b, h], P2[b, h], V[b, h], float(tau[h]), lam)
    return out


def decode_bar(p1, p2, v, cache_P2, cache_V, lens, tau, lam=0.0):
    """Elementwise bound [B, H, d_h] on one fp32 decode step: the forward's
    bar for the row of the new token (position L_b + 1), whose keys are the
    cached ones followed by the token itself."""
    B, H, d = p1.shape
    k = 1.0 / math.sqrt(d)
    out = np.empty(p1.shape)
    for b in range(B):
        L = int(np.clip(lens[b], 0, cache_P2.shape[2]))
        i = L + 1
        for h in range(H):
            tau_h = float(tau[h])
            q = p1[b, h]
            keys = np.concatenate([cache_P2[b, h, :L], p2[b, h][None]])
            vv = np.concatenate([cache_V[b, h, :L], v[b, h][None]])
            u = keys @ q * k
            A = np.abs(keys) @ np.abs(q) * k
            dU = U_RND * (LAM * math.sqrt(d) * A + 2.0 * np.abs(u))
            E = O.silu(u[:L])
            m = float(np.max(E)) if L else 0.0
            S = float(O.sigmoid(np.array([u[L] / tau_h]))[0])
            r = np.concatenate([E - lam * math.log(i), [S]])
            w = np.exp(r - np.max(r))
            F = w / w.sum()
            eps = np.empty(i)
            eps[:L] = 1.1 * dU[:L] + U_RND * (8.0 * np.abs(E) + 2.0 * abs(m) + 2.0 * abs(lam) * math.log(i) + 4.0)
            eps[L] = 0.25 * (dU[L] + 2.0 * U_RND * abs(u[L])) / tau_h + 6.0 * U_RND
            alpha = LAM * math.sqrt(2.0 * i) * U_RND + 2.0 * U_RND
            y = F @ vv
            out[b, h] = ((F * eps) @ np.abs(vv - y) + alpha * (F @ np.abs(vv) + np.abs(y))
                         + 3.0 * U_RND * np.abs(y))
    return out


def bwd_head_bars(p1, p2, v, tau, lam, dy):
    """Elementwise bounds on an fp32 backward of one head that recomputes F
    from the stored fp32 LSE and uses the stored fp32 Y: a dict with dP1, dP2,
    dV ([T, d_h]) and dtau, dlam (scalars)."""
    T, d = p1.shape
    k = 1.0 / math.sqrt(d)
    t = _head_terms(p1, p2, tau, lam)
    U, dU, F, eps, alpha, below = t["U"], t["dU"], t["F"], t["eps"], t["alpha"], t["below"]
    diag = np.arange(T)
    Y = F @ v
    lse = O.row_lse(p1, p2, tau, lam)
    dlse = np.sum(F * eps, axis=1) + alpha + U_RND * np.abs(lse)
    phi = np.where(F > 0, eps + dlse[:, None], 0.0)
    beta = LAM * math.sqrt(T) * U_RND
    dF = dy @ v.T
    D = np.sum(dy * Y, axis=1)
    dR = F * (dF - D[:, None])
    dD = (np.sum(eps * np.abs(dR), axis=1)
          + alpha * np.sum(np.abs(dy) * (F @ np.abs(v) + np.abs(Y)), axis=1)
          + (LAM * math.sqrt(d) + 3.0) * U_RND * np.sum(np.abs(dy * Y), axis=1))
    eta = LAM * math.sqrt(d) * U_RND * (np.abs(dy) @ np.abs(v).T)
    ddR = phi * np.abs(dR) + F * (eta + dD[:, None]) + 2.0 * U_RND * np.abs(dR)
    s = O.sigmoid(U[diag, diag] / tau)
    g = np.where(below, O.silu_grad(U), 0.0)
    g[diag, diag] = s * (1.0 - s) / tau
    gp = np.where(below, 0.5, 0.0)
    gp[diag, diag] = 0.1 / tau ** 2
    dg = gp * dU + 6.0 * U_RND * np.abs(g)
    dUg = dR * g
    ddU = ddR * np.abs(g) + np.abs(dR) * dg + U_RND * np.abs(dUg)
    ddU = np.where(below | (diag[:, None] == diag[None, :]), ddU, 0.0)
    out = {}
    out["dV"] = (F * (phi + beta)).T @ np.abs(dy)
    out["dP1"] = k * ((ddU + (beta + 2.0 * U_RND) * np.abs(dUg)) @ np.abs(p2))
    out["dP2"] = k * ((ddU + (beta + 2.0 * U_RND) * np.abs(dUg)).T @ np.abs(p1))
    Ud = U[diag, diag]
    q = -s * (1.0 - s) * Ud / tau ** 2
    dq = (0.1 * np.abs(Ud) + 0.25) / tau ** 2
    dRd, ddRd = dR[diag, diag], ddR[diag, diag]
    out["dtau"] = float(np.sum(ddRd * np.abs(q) + np.abs(dRd) * (dq * dU[diag, diag] + 6.0 * U_RND * np.abs(q)))
                        + beta * np.sum(np.abs(dRd * q)))
    logi = t["logi"]
    out["dlam"] = float(np.sum(logi * (ddRd + (beta + 2.0 * U_RND) * np.abs(dRd))))
    return out


def bwd_bars(P1, P2, V, tau, lam, dY):
    """bwd_head_bars over [B, H, T, d_h]: dP1, dP2, dV elementwise, dtau [H]
    (summed over the batch like dtau itself) and dlam (summed over all)."""
    B, H = P1.shape[:2]
    out = dict(dP1=np.empty(P1.shape), dP2=np.empty(P1.shape), dV=np.empty(P1.shape),
               dtau=np.zeros(H), dlam=0.0)
    for b in range(B):
        for h in range(H):
            r = bwd_head_bars(P1[b, h], P2[b, h], V[b, h], float(tau[h]), lam, dY[b, h])
            for key in ("dP1", "dP2", "dV"):
                out[key][b, h] = r[key]
            out["dtau"][h] += r["dtau"]
            out["dlam"] += r["dlam"]
    return out


def excess(got, ref, bar):
    """max |got - ref| / bar over all elements (0/0 counts as 0: where the
    bound is exactly zero, the exact result is required)."""
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    bar = np.broadcast_to(np.asarray(bar, np.float64), err.shape)
    r = np.divide(err, bar, out=np.where(err > 0, np.inf, 0.0), where=bar > 0)
    return float(np.max(r)) if r.size else 0.0

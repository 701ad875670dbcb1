"""Plain fp64 CPU oracle for the Linear Relation forward.

TEST INFRASTRUCTURE ONLY, under the same rules as ``relation_oracle``: only
the test suite, the smoke check and the benchmark's CPU-baseline leg may use
it; it shares no code with the HIP kernels.

Source: "Ask Self, Ask Others: Relation Is All You Need", abbreviated [paper],
Sec. 5.2 Eq. (15)-(17) and App. A.4. Per head, for t = 1..T (rows of P1, P2, I
are tokens; P1 / P2 are the relation coordinates after RoPE, I the mixed
information state I~, alpha the channel-wise retention in (0, 1]^{d_h}):
  S_t   = sigmoid(p1_t . p2_t / (tau sqrt(d_h)))                Eq. (15)
  p^1_t = p1_t / ||p1_t||,  p^2_t = p2_t / ||p2_t||             Eq. (15)
  C_0 = 0 (d_h x d_h);  C-_t = Diag(alpha_t) C_{t-1}            Eq. (17), A.4.2
  E_t = S_t (C-_t)^T p^1_t;  Y_t = I_t + E_t                    (read ...)
  C_t = C-_t + S_t p^2_t I_t^T                                  (... then write)
The retention alpha is an input (its parameterisation, Eq. (16), needs learned
weights). ``linear_relation_head`` is the recurrence itself; the unrolled
form of App. A.4.4-A.4.5, ``linear_relation_unrolled``, is a second route used
only to pin it.

Reading: a zero row of P1 or P2 has no direction; its normalised coordinate
is taken as 0 (the state neither reads nor writes along it).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["normalize_rows", "self_relation", "linear_relation_head", "linear_relation_fwd",
           "linear_relation_unrolled"]


def normalize_rows(x):
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def self_relation(p1, p2, tau):
    d = p1.shape[-1]
    u = np.sum(np.asarray(p1, np.float64) * np.asarray(p2, np.float64), axis=-1) / (float(tau) * math.sqrt(d))
    return 1.0 / (1.0 + np.exp(-u))


def linear_relation_head(p1, p2, I, alpha, tau, return_state=False):
    """Y [T, d] of one head by the recurrence (Eq. (17)); optionally C_T."""
    I = np.asarray(I, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    T, d = I.shape
    S = self_relation(p1, p2, tau)
    q, k = normalize_rows(p1), normalize_rows(p2)
    C = np.zeros((d, d))
    Y = np.empty((T, d))
    for t in range(T):
        C = alpha[t][:, None] * C                   # C-_t = Diag(alpha_t) C_{t-1}
        Y[t] = I[t] + S[t] * (C.T @ q[t])           # Ask Others, Answer
        C = C + S[t] * np.outer(k[t], I[t])         # Become Others
    return (Y, C) if return_state else Y


def linear_relation_fwd(P1, P2, I, alpha, tau, return_state=False):
    """[B, H, T, d] inputs, alpha [B, H, T, d], tau [H]; returns Y (and C_T [B, H, d, d])."""
    B, H, T, d = np.shape(P1)
    Y = np.empty((B, H, T, d))
    C = np.empty((B, H, d, d))
    for b in range(B):
        for h in range(H):
            Y[b, h], C[b, h] = linear_relation_head(P1[b, h], P2[b, h], I[b, h], alpha[b, h], tau[h], True)
    return (Y, C) if return_state else Y


def linear_relation_unrolled(p1, p2, I, alpha, tau):
    """Second route ([paper] App. A.4.5): E_t = S_t sum_{j<t} S_j
    (p^2_j^T (prod_{u=j+1..t} D_u) p^1_t) I_j, summed term by term."""
    I = np.asarray(I, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    T, d = I.shape
    S = self_relation(p1, p2, tau)
    q, k = normalize_rows(p1), normalize_rows(p2)
    Y = I.copy()
    for t in range(T):
        for j in range(t):
            decay = np.prod(alpha[j + 1: t + 1], axis=0)      # D_t D_{t-1} ... D_{j+1}
            Y[t] += S[t] * S[j] * float(np.sum(k[j] * decay * q[t])) * I[j]
    return Y

"""Plain fp64 CPU oracle for the model-side pre-steps of Multi-Head Relation:
rotary position encoding (RoPE) of the relation coordinates P1, P2 and Givens
mixing of the information heads.

TEST INFRASTRUCTURE ONLY, under the same rules as ``relation_oracle``: only
the test suite, the smoke check and the benchmark's CPU-baseline leg may use
it; it shares no code with the HIP kernels.

Source: "Ask Self, Ask Others: Relation Is All You Need", abbreviated [paper].
  Givens block ([paper] Eq. (4), App. A.2.2): for an adjacent head pair (a, b)
  and the pair's angle t,
      I~(a) = cos t I(a) - sin t I(b),     I~(b) = sin t I(a) + cos t I(b),
  one scalar angle acting on all d_h channels of the pair (an orthogonal map).
  Alternating pairing ([paper] App. A.2.3), one-based heads, H even:
      M_A = {(1, 2), (3, 4), ..., (H-1, H)},   M_B = {(2, 3), (4, 5), ..., (H, 1)},
  alternating across layers; H / 2 angles per layer.
  RoPE ([paper] Sec. 6, App. B.3): full head dimension, base 10^4, applied to P1
  and P2 before the evidence; the information branch is not rotated.

Readings (the pages leave these open):
  * angle k of a pairing belongs to its k-th pair in the order listed above;
  * the rotary pairs follow one of two conventions, both provided:
    "interleaved" rotates (x_{2k}, x_{2k+1}) and "half" rotates (x_k, x_{k+d/2}),
    each by the angle pos * base^(-2k / d_h), k = 0 .. d_h/2 - 1
    (x' = x_a cos - x_b sin, x_b' = x_a sin + x_b cos);
  * pos is the zero-based token index, offset per sequence by pos0[b].
"""
from __future__ import annotations

import numpy as np

from oracle import relation_oracle as RO

__all__ = ["rope", "head_pairs", "givens_mix", "prestep", "relation_fwd_model"]

MODES = ("none", "interleaved", "half")


def rope(x, pos, base=1e4, mode="interleaved"):
    """Rotate the rows of x [..., T, d] at positions pos [T] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    if mode == "none":
        return x.copy()
    d = x.shape[-1]
    k = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * k / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    if mode == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
    elif mode == "half":
        a, b = x[..., : d // 2], x[..., d // 2:]
        out[..., : d // 2] = a * c - b * s
        out[..., d // 2:] = a * s + b * c
    else:
        raise ValueError(mode)
    return out


def head_pairs(H, pairing):
    """Zero-based (a, b) head pairs of pairing "A" or "B" ([paper] App. A.2.3)."""
    if H % 2:
        raise ValueError("Givens pairing needs an even number of heads")
    if pairing == "A":
        return [(2 * k, 2 * k + 1) for k in range(H // 2)]
    if pairing == "B":
        return [(2 * k + 1, (2 * k + 2) % H) for k in range(H // 2)]
    raise ValueError(pairing)


def givens_mix(I, theta, pairing):
    """Mix information heads I [B, H, T, d] in pairs ([paper] Eq. (4), App. A.2.2)."""
    I = np.asarray(I, dtype=np.float64)
    out = I.copy()
    for k, (a, b) in enumerate(head_pairs(I.shape[1], pairing)):
        c, s = np.cos(float(theta[k])), np.sin(float(theta[k]))
        out[:, a] = c * I[:, a] - s * I[:, b]
        out[:, b] = s * I[:, a] + c * I[:, b]
    return out


def prestep(P1, P2, I, pos0=None, base=1e4, mode="interleaved", theta=None, pairing="A"):
    """RoPE on P1 and P2 (positions pos0[b] + t) and Givens mixing of I
    (skipped when theta is None). Inputs [B, H, T, d]; returns fp64 copies."""
    P1 = np.asarray(P1, dtype=np.float64)
    P2 = np.asarray(P2, dtype=np.float64)
    B, H, T, _ = P1.shape
    off = np.zeros(B, dtype=np.int64) if pos0 is None else np.asarray(pos0, dtype=np.int64)
    P1o = np.empty_like(P1)
    P2o = np.empty_like(P2)
    for b in range(B):
        pos = off[b] + np.arange(T)
        P1o[b] = rope(P1[b], pos, base, mode)
        P2o[b] = rope(P2[b], pos, base, mode)
    Io = np.asarray(I, dtype=np.float64).copy() if theta is None else givens_mix(I, theta, pairing)
    return P1o, P2o, Io


def relation_fwd_model(P1, P2, I, tau, lam=0.0, pos0=None, base=1e4, mode="interleaved", theta=None,
                       pairing="A"):
    """The relation forward on raw projections: the pre-steps, then Eq. (1)-(3)."""
    a, b, c = prestep(P1, P2, I, pos0, base, mode, theta, pairing)
    return RO.relation_fwd(a, b, c, tau, lam)

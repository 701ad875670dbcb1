"""Arbitrary-precision brute force for tiny heads (test infrastructure only).

Evaluates the definition of "Ask Self, Ask Others: Relation Is All You Need"
Eq. (1)-(3) with mpmath at 50 significant digits, in pure Python loops, without
the max-shift used by the fp64 oracle: every weight is exp(R_ij) divided by the
row total, which is safe at this precision for the small magnitudes used.
Intended for T <= 8, d_h <= 4.
"""
from __future__ import annotations

import mpmath as mp


def brute_head(p1, p2, v, tau, lam=0.0, dps=50):
    """p1, p2, v: nested sequences [T][d]; returns [T][d_v] as mpf."""
    with mp.workdps(dps):
        T = len(p1)
        d = len(p1[0])
        root = mp.sqrt(d)
        out = []
        for r in range(T):
            i = r + 1
            weights = []
            for c in range(i):
                u = mp.fsum(mp.mpf(p1[r][k]) * mp.mpf(p2[c][k]) for k in range(d)) / root
                if c == r:
                    logit = 1 / (1 + mp.exp(-u / mp.mpf(tau)))
                else:
                    logit = u / (1 + mp.exp(-u)) - mp.mpf(lam) * mp.log(i)
                weights.append(mp.exp(logit))
            total = mp.fsum(weights)
            row = []
            for k in range(len(v[0])):
                row.append(mp.fsum(weights[c] * mp.mpf(v[c][k]) for c in range(i)) / total)
            out.append(row)
        return out

"""Pins of the derived fp32 error bars (tests/fp32_bars.py) on the CPU.

The bars replace a fixed tolerance in the large-evidence GPU tests, so they
are checked from both sides here:
  - they admit independent fp32 evaluations of the operator (the definition
    in torch fp32 with autograd, and a key-by-key online scan in numpy fp32
    that accumulates O and l one term at a time, as the row-scan kernels do);
  - they are not vacuous: mistakes of the size fp32 must rule out (the
    Exchange weights or the key operand P2 rounded to bf16, one rescaling of
    the running maximum skipped) exceed them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import relation_oracle as O
from tests import fp32_bars as FB


def _large_inputs(D, T=160, H=2, seed=0):
    """The large-evidence recipe of the GPU tests: P1, P2 ~ base + 0.4 N(0,1)
    with base^2 sqrt(d_h) = 30, so U_ij ~ 30 (up to ~45); V ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    base = np.float32(np.sqrt(30.0 / np.sqrt(D)))
    P1 = (base + 0.4 * rng.standard_normal((1, H, T, D))).astype(np.float32)
    P2 = (base + 0.4 * rng.standard_normal((1, H, T, D))).astype(np.float32)
    V = rng.standard_normal((1, H, T, D)).astype(np.float32)
    dY = rng.standard_normal((1, H, T, D)).astype(np.float32)
    return P1, P2, V, dY, np.array([1.0, 0.5], np.float32)


def _torch_fp32(P1, P2, V, tau, lam, dY=None):
    """The definition ([paper] Eq. (1)-(3)) in torch fp32, with autograd."""
    p1, p2, v = (torch.tensor(x, requires_grad=True) for x in (P1, P2, V))
    t = torch.tensor(tau, requires_grad=True)
    lm = torch.tensor(np.float32(lam), requires_grad=True)
    T, D = P1.shape[-2:]
    U = p1 @ p2.transpose(-1, -2) / math.sqrt(D)
    i = torch.arange(1, T + 1, dtype=torch.float32)
    E = torch.nn.functional.silu(U) - lm * torch.log(i)[:, None]
    S = torch.sigmoid(torch.diagonal(U, dim1=-2, dim2=-1) / t[None, :, None])
    below = torch.tril(torch.ones(T, T, dtype=torch.bool), -1)
    R = torch.where(below, E, torch.full_like(E, -float("inf")))
    R = torch.where(torch.eye(T, dtype=torch.bool), torch.diag_embed(S), R)
    F = torch.softmax(R, dim=-1)
    Y = F @ v
    if dY is None:
        return Y.detach().numpy().astype(np.float64)
    dy = torch.tensor(dY)
    (Y * dy).sum().backward()
    # dlambda as the kernels form it, from the diagonal of dR (each row of dR
    # sums to zero): sum_i log i dR_ii, dR = F (dY V^T - D)
    with torch.no_grad():
        dR = F * (dy @ v.transpose(-1, -2) - (dy * Y).sum(-1, keepdim=True))
        dlam = float((torch.log(i) * torch.diagonal(dR, dim1=-2, dim2=-1)).sum())
    return dict(dP1=p1.grad.numpy(), dP2=p2.grad.numpy(), dV=v.grad.numpy(),
                dtau=t.grad.numpy(), dlam=dlam)


def _scan_fp32(p1, p2, v, tau, lam, round_w=None, skip_rescale_at=None):
    """Key-by-key online scan in numpy fp32 (one head): Exchange first, Self
    once at the end ([paper] Eq. (12)-(14)). round_w / skip_rescale_at plant
    mistakes for the rejection pins."""
    f = np.float32
    T, D = p1.shape
    k = f(1.0 / math.sqrt(D))
    Y = np.empty((T, D), np.float32)
    for r in range(T):
        m, l, z = f(-np.inf), f(0.0), np.zeros(D, np.float32)
        for j in range(r):
            u = f(np.dot(p1[r], p2[j])) * k
            e = u / (f(1.0) + np.exp(-u))
            if e > m:
                s = f(0.0) if m == -np.inf else np.exp(m - e)
                if skip_rescale_at is not None and (r, j) == skip_rescale_at:
                    s = f(1.0)
                l, z, m = l * s, z * s, e
            w = np.exp(e - m)
            if round_w is not None:
                w = round_w(w)
            l = l + w
            z = z + w * v[j]
        uii = f(np.dot(p1[r], p2[r])) * k
        S = f(1.0) / (f(1.0) + np.exp(-uii / f(tau)))
        if r == 0:
            Y[r] = v[r]
            continue
        mc = m - f(lam) * f(math.log(r + 1))
        M = max(mc, S)
        a, c = np.exp(S - M), np.exp(mc - M)
        Y[r] = (a * v[r] + c * z) / (a + c * l)
    return Y.astype(np.float64)


def _bf16(x):
    return float(torch.tensor(float(x), dtype=torch.float32).to(torch.bfloat16).float())


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_bar_admits_fp32_definition(D):
    P1, P2, V, _, tau = _large_inputs(D)
    ref = O.relation_fwd(*(x.astype(np.float64) for x in (P1, P2, V)), tau.astype(np.float64), 0.5)
    bar = FB.fwd_bar(*(x.astype(np.float64) for x in (P1, P2, V)), tau.astype(np.float64), 0.5)
    err = np.abs(_torch_fp32(P1, P2, V, tau, 0.5) - ref)
    assert FB.excess(err, 0.0, bar) <= 1.0
    # not vacuous: the bar stays within a few hundred times the error it covers
    assert np.max(bar) <= 300 * np.max(err), (np.max(bar), np.max(err))


def test_fwd_bar_admits_fp32_scan_and_rejects_planted_mistakes():
    D, T = 128, 96
    P1, P2, V, _, tau = _large_inputs(D, T=T, H=1, seed=3)
    p1, p2, v = P1[0, 0], P2[0, 0], V[0, 0]
    f64 = lambda x: x.astype(np.float64)
    ref = O.relation_head(f64(p1), f64(p2), f64(v), float(tau[0]), 0.5)
    bar = FB.fwd_head_bar(f64(p1), f64(p2), f64(v), float(tau[0]), 0.5)
    ok = np.abs(_scan_fp32(p1, p2, v, tau[0], 0.5) - ref)
    assert FB.excess(ok, 0.0, bar) <= 1.0
    # the Exchange weights rounded to bf16 (what the bf16 path does): rejected
    bad = np.abs(_scan_fp32(p1, p2, v, tau[0], 0.5, round_w=lambda w: np.float32(_bf16(w))) - ref)
    assert np.any(bad > bar)
    # one rescaling of the running maximum skipped: rejected
    row = T - 1
    E = O.silu(O.evidence(f64(p1), f64(p2))[row, :row])
    j = int(np.flatnonzero(E > np.maximum.accumulate(np.concatenate([[-np.inf], E[:-1]])))[-1])
    bad = np.abs(_scan_fp32(p1, p2, v, tau[0], 0.5, skip_rescale_at=(row, j)) - ref)
    assert np.any(bad > bar)
    # P2 read at bf16 precision (an fp32 path that silently narrows a key
    # operand): rejected
    p2b = torch.from_numpy(p2).to(torch.bfloat16).double().numpy()
    bad = np.abs(O.relation_head(f64(p1), p2b, f64(v), float(tau[0]), 0.5) - ref)
    assert np.any(bad > bar)


def test_decode_bar_is_the_forward_bar_of_the_last_row():
    """decode_bar computes one row on its own; it must equal the forward bar
    of that row of the full sequence (cache followed by the new token)."""
    D, L = 64, 70
    P1, P2, V, _, tau = _large_inputs(D, T=L + 1, H=2, seed=5)
    f64 = lambda x: x.astype(np.float64)
    full = FB.fwd_bar(f64(P1), f64(P2), f64(V), f64(tau), 0.5)[0, :, L]
    dec = FB.decode_bar(f64(P1[:, :, L]), f64(P2[:, :, L]), f64(V[:, :, L]), f64(P2), f64(V),
                        np.array([L]), f64(tau), 0.5)[0]
    np.testing.assert_allclose(dec, full, rtol=1e-12, atol=0)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_bars_admit_fp32_definition(D):
    P1, P2, V, dY, tau = _large_inputs(D, T=128)
    f64 = lambda x: x.astype(np.float64)
    ref = O.relation_bwd(f64(P1), f64(P2), f64(V), f64(tau), 0.5, f64(dY))
    bars = FB.bwd_bars(f64(P1), f64(P2), f64(V), f64(tau), 0.5, f64(dY))
    got = _torch_fp32(P1, P2, V, tau, 0.5, dY)
    # P2 read at bf16 precision, planted in the oracle: every gradient tensor
    # moves past its bar somewhere
    p2b = torch.from_numpy(P2).to(torch.bfloat16).double().numpy()
    bad = O.relation_bwd(f64(P1), p2b, f64(V), f64(tau), 0.5, f64(dY))
    for n, key in enumerate(("dP1", "dP2", "dV")):
        err = np.abs(got[key] - ref[n])
        assert FB.excess(err, 0.0, bars[key]) <= 1.0, key
        assert np.any(np.abs(bad[n] - ref[n]) > bars[key]), key
    assert np.all(np.abs(got["dtau"] - ref[3]) <= bars["dtau"])
    # dlambda: the diagonal form of the oracle's dR (see the GPU test for why)
    logi = np.log(np.arange(1, P1.shape[2] + 1))
    dlam = sum(float(np.sum(logi * O.relation_head_bwd(f64(P1[0, h]), f64(P2[0, h]), f64(V[0, h]), float(tau[h]),
                                                     0.5, f64(dY[0, h]), return_terms=True)[5]["dR_self"]))
               for h in range(P1.shape[1]))
    assert abs(got["dlam"] - dlam) <= bars["dlam"]


def test_excess_treats_a_zero_bound_as_exact():
    assert FB.excess([1.0, 2.0], [1.0, 2.0], [0.0, 0.0]) == 0.0
    assert FB.excess([1.0, 2.5], [1.0, 2.0], [0.0, 1.0]) == 0.5
    assert FB.excess([1.0 + 1e-300, 2.0], [1.0, 2.0], [0.0, 1.0]) == 0.0   # 1 + 1e-300 == 1
    assert FB.excess([1.5, 2.0], [1.0, 2.0], [0.0, 1.0]) == np.inf

"""Pins for the oracle's gradients (``relation_head_bwd`` / ``relation_bwd``)
and its per-row log normaliser (``row_lse``).

The pages define only the forward operator ("Ask Self, Ask Others: Relation Is
All You Need", Eq. (1)-(3)); the gradients are the calculus of that definition.
None of these pins retypes the oracle's chain rule:
  * central finite differences of the oracle's *forward* (fp64) for every
    input, tau and lambda;
  * reverse-mode differentiation by torch.autograd (CPU, fp64) of a separate
    torch transcription of Eq. (1)-(3) -- the derivative is produced
    mechanically, not by the hand-written chain rule;
  * closed forms: a single token (Y_1 = V_1), constant information rows (Y no
    longer depends on P1, P2, tau, lambda), and the paper's partition
    Z_i = e^{S_i} + e^{A_i} (Eq. (6)-(7)) for LSE.
Mistakes each pin is meant to catch (a dropped 1/sqrt(d_h) or 1/tau, the
softmax-backward correction D_i left out, SiLU' taken as sigmoid, dP1/dP2
swapped, a zero-based count index in dlambda, tau gradients not summed over
the batch) are noted per test.
"""
import math

import numpy as np
import pytest
import torch

from oracle import relation_oracle as O


def _head(rng, T, d, scale=1.0):
    return tuple(rng.standard_normal((T, d)) * scale for _ in range(4))


def _fd(f, x, eps=1e-6):
    """Central differences of scalar f at array x (copied per coordinate)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        a = x.copy(); a[i] += eps
        b = x.copy(); b[i] -= eps
        g[i] = (f(a) - f(b)) / (2 * eps)
    return g


@pytest.mark.parametrize("T,d,tau,lam,seed", [(2, 1, 1.0, 0.0, 0), (3, 3, 0.5, 0.5, 1),
                                              (5, 4, 2.0, 0.0, 2), (7, 2, 1.3, 0.5, 3)])
def test_gradients_match_central_differences(T, d, tau, lam, seed):
    """Every gradient against finite differences of the forward alone (catches
    any slip in the chain rule: missing D_i, wrong SiLU', missing 1/tau or
    1/sqrt(d_h), transposed dU)."""
    rng = np.random.default_rng(seed)
    p1, p2, v, dy = _head(rng, T, d)
    g = O.relation_head_bwd(p1, p2, v, tau, lam, dy)

    def loss(P1=p1, P2=p2, V=v, ta=tau, la=lam):
        return float(np.sum(O.relation_head(P1, P2, V, ta, la) * dy))

    np.testing.assert_allclose(g[0], _fd(lambda x: loss(P1=x), p1), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g[1], _fd(lambda x: loss(P2=x), p2), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g[2], _fd(lambda x: loss(V=x), v), rtol=1e-6, atol=1e-8)
    eps = 1e-6
    assert math.isclose(g[3], (loss(ta=tau + eps) - loss(ta=tau - eps)) / (2 * eps), rel_tol=1e-6, abs_tol=1e-8)
    assert math.isclose(g[4], (loss(la=lam + eps) - loss(la=lam - eps)) / (2 * eps), rel_tol=1e-6, abs_tol=1e-8)


def _torch_forward(p1, p2, v, tau, lam):
    """Eq. (1)-(3) in torch ops (fp64), differentiated by autograd below."""
    T, d = p1.shape
    U = p1 @ p2.T / math.sqrt(d)
    i = torch.arange(1, T + 1, dtype=torch.float64)
    E = U * torch.sigmoid(U) - lam * torch.log(i)[:, None]
    S = torch.sigmoid(torch.diagonal(U) / tau)
    R = torch.where(torch.ones(T, T, dtype=torch.bool).tril(-1), E, torch.full_like(E, -math.inf))
    R = torch.where(torch.eye(T, dtype=torch.bool), torch.diag_embed(S), R)
    return torch.softmax(R, dim=1) @ v


@pytest.mark.parametrize("seed", [4, 5, 6])
def test_gradients_match_autograd(seed):
    """Reverse-mode autograd of a torch transcription of the definition."""
    rng = np.random.default_rng(seed)
    T, d = 9, 5
    p1, p2, v, dy = _head(rng, T, d, scale=1.5)
    tau, lam = 0.8, 0.5
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (p1, p2, v)]
    ta = torch.tensor(tau, dtype=torch.float64, requires_grad=True)
    la = torch.tensor(lam, dtype=torch.float64, requires_grad=True)
    y = _torch_forward(t[0], t[1], t[2], ta, la)
    np.testing.assert_allclose(y.detach().numpy(), O.relation_head(p1, p2, v, tau, lam), rtol=1e-12, atol=1e-12)
    (y * torch.tensor(dy)).sum().backward()
    g = O.relation_head_bwd(p1, p2, v, tau, lam, dy)
    for k in range(3):
        np.testing.assert_allclose(g[k], t[k].grad.numpy(), rtol=1e-10, atol=1e-12)
    assert math.isclose(g[3], ta.grad.item(), rel_tol=1e-10, abs_tol=1e-12)
    assert math.isclose(g[4], la.grad.item(), rel_tol=1e-10, abs_tol=1e-12)


def test_single_token_passes_the_gradient_to_v_only():
    """T = 1: Y_1 = V_1 ([paper] App. A.1.7), so dV = dY and nothing else moves."""
    rng = np.random.default_rng(7)
    p1, p2, v, dy = _head(rng, 1, 6)
    dP1, dP2, dV, dtau, dlam = O.relation_head_bwd(p1, p2, v, 1.7, 0.5, dy)
    np.testing.assert_array_equal(dV, dy)
    assert np.max(np.abs(dP1)) < 1e-15 and np.max(np.abs(dP2)) < 1e-15
    assert abs(dtau) < 1e-15 and abs(dlam) < 1e-15


def test_constant_information_rows_stop_all_other_gradients():
    """Rows of F sum to 1, so with every V_j equal to c, Y_i = c whatever P1,
    P2, tau, lambda are: their gradients vanish (up to rounding) while dV is
    the column sums of F spread over the rows."""
    rng = np.random.default_rng(8)
    T, d = 12, 4
    p1, p2, _, dy = _head(rng, T, d, scale=2.0)
    v = np.tile(rng.standard_normal(d), (T, 1))
    dP1, dP2, dV, dtau, dlam = O.relation_head_bwd(p1, p2, v, 0.9, 0.5, dy)
    assert np.max(np.abs(dP1)) < 1e-12 and np.max(np.abs(dP2)) < 1e-12
    assert abs(dtau) < 1e-12 and abs(dlam) < 1e-12
    np.testing.assert_allclose(dV.sum(axis=0), dy.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_gradients_are_linear_in_the_upstream_gradient():
    rng = np.random.default_rng(9)
    p1, p2, v, dy1 = _head(rng, 6, 3)
    dy2 = rng.standard_normal(dy1.shape)
    g1 = O.relation_head_bwd(p1, p2, v, 1.1, 0.5, dy1)
    g2 = O.relation_head_bwd(p1, p2, v, 1.1, 0.5, dy2)
    g = O.relation_head_bwd(p1, p2, v, 1.1, 0.5, dy1 - 3.0 * dy2)
    for k in range(5):
        np.testing.assert_allclose(g[k], np.asarray(g1[k]) - 3.0 * np.asarray(g2[k]), rtol=1e-10, atol=1e-12)


def test_multihead_gradients_sum_tau_over_batch_and_lambda_over_everything():
    """tau is one value per head shared by the batch, lambda one scalar: their
    gradients are sums of the per-(b, h) ones; the tensors stay per head."""
    rng = np.random.default_rng(10)
    B, H, T, d = 2, 3, 5, 4
    P1, P2, V, dY = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    tau = np.array([0.6, 1.0, 1.7])
    dP1, dP2, dV, dtau, dlam = O.relation_bwd(P1, P2, V, tau, 0.5, dY)
    want_tau = np.zeros(H)
    want_lam = 0.0
    for b in range(B):
        for h in range(H):
            g = O.relation_head_bwd(P1[b, h], P2[b, h], V[b, h], tau[h], 0.5, dY[b, h])
            np.testing.assert_array_equal(dP1[b, h], g[0])
            want_tau[h] += g[3]
            want_lam += g[4]
    np.testing.assert_allclose(dtau, want_tau, rtol=1e-14)
    assert math.isclose(dlam, want_lam, rel_tol=1e-14)


def test_future_gradients_do_not_reach_the_past():
    """Row i's query gradient dP1_i sees dY only through row i (Y_i is the only
    output p1_i feeds, [paper] Eq. (3)): with dY zero on rows < k, dP1 is
    exactly zero on those rows."""
    rng = np.random.default_rng(11)
    p1, p2, v, dy = _head(rng, 10, 3)
    dy[:4] = 0.0
    dP1 = O.relation_head_bwd(p1, p2, v, 1.0, 0.5, dy)[0]
    assert np.max(np.abs(dP1[:4])) == 0.0


@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_row_lse_is_the_paper_partition(lam):
    """LSE_i = log(e^{S_i} + e^{A_i}) with the Exchange log-mass A_i of
    Eq. (6) ([paper] Eq. (6)-(7)); row 1 has A_1 = -inf so LSE_1 = S_1."""
    rng = np.random.default_rng(12)
    p1, p2, v, _ = _head(rng, 8, 4, scale=1.5)
    fz = O.factorized_head(p1, p2, v, 1.2, lam)
    want = np.logaddexp(fz["S"], fz["A"])
    np.testing.assert_allclose(O.row_lse(p1, p2, 1.2, lam), want, rtol=1e-13, atol=1e-13)
    assert O.row_lse(p1, p2, 1.2, lam)[0] == pytest.approx(fz["S"][0], abs=1e-15)


@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_row_terms_sum_to_the_scalars_and_rows_of_dR_sum_to_zero(lam):
    """The per-row terms add up to dtau / dlambda, and since every row of F
    sums to one, sum_j dR_ij = D_i - D_i = 0: row i's dlambda share
    -log i sum_{j<i} dR_ij equals log i dR_ii (the form the kernels use)."""
    rng = np.random.default_rng(13)
    p1, p2, v, dy = _head(rng, 11, 4, scale=1.3)
    *g, terms = O.relation_head_bwd(p1, p2, v, 0.7, lam, dy, return_terms=True)
    assert math.isclose(np.sum(terms["tau_terms"]), g[3], rel_tol=1e-12, abs_tol=1e-14)
    assert math.isclose(np.sum(terms["lam_terms"]), g[4], rel_tol=1e-12, abs_tol=1e-14)
    log_i = np.log(np.arange(1, 12))
    np.testing.assert_allclose(terms["lam_terms"], log_i * terms["dR_self"], rtol=1e-9, atol=1e-13)
    # and the Self weight is e^{S_i - LSE_i}
    np.testing.assert_allclose(terms["F_self"], np.exp(terms["S"] - O.row_lse(p1, p2, 0.7, lam)), rtol=1e-12)


@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_sampled_gradients_equal_the_materialised_ones(lam):
    """The row / column route for large T agrees with the materialised
    backward (itself pinned above) on every row and column, with a block size
    that does not divide T."""
    rng = np.random.default_rng(14)
    T, d = 37, 5
    p1, p2, v, dy = _head(rng, T, d, scale=1.2)
    full = O.relation_head_bwd(p1, p2, v, 0.8, lam, dy)
    rows = list(range(T))
    got = O.relation_head_bwd_sampled(p1, p2, v, 0.8, lam, dy, rows, rows, block=8)
    np.testing.assert_allclose(got["dP1"], full[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dP2"], full[1], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dV"], full[2], rtol=1e-10, atol=1e-12)
    assert math.isclose(got["dtau"], full[3], rel_tol=1e-10, abs_tol=1e-12)
    np.testing.assert_allclose(got["lse"], O.row_lse(p1, p2, 0.8, lam), rtol=1e-12)
    np.testing.assert_allclose(got["Y"], O.relation_head(p1, p2, v, 0.8, lam), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_dp1_rows_equal_the_materialised_ones(lam):
    """The row-only dP1 route (for lengths where no T x T matrix or full
    forward pass is affordable) agrees with the materialised backward on
    every row, the first (Self only) and the last included."""
    rng = np.random.default_rng(15)
    T, d = 29, 6
    p1, p2, v, dy = _head(rng, T, d, scale=1.3)
    full = O.relation_head_bwd(p1, p2, v, 0.7, lam, dy)
    got = O.relation_head_dp1_rows(p1, p2, v, 0.7, lam, dy, list(range(T)))
    np.testing.assert_allclose(got, full[0], rtol=1e-10, atol=1e-12)

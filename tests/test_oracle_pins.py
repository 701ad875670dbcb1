"""Pins for the CPU oracle, checked against facts the paper and mathematics fix.

None of these retypes the oracle's own formula. Each pin comes from an
independent statement: closed forms derived by hand from "Ask Self, Ask Others:
Relation Is All You Need" Eq. (1)-(3), the identities of its Sec. 4.2 / App. A.1,
the exactness of the tiled scan (Sec. 5.1, App. A.3.5), the first-token boundary
(App. A.1.7), the projected cache (Eq. (18), App. A.5), a regime in which the
operator reduces to textbook strictly-causal softmax attention, and the
arbitrary-precision brute force of ``oracle.brute_mp`` on tiny heads.

Mistakes each pin is meant to catch (dropped 1/sqrt(d_h), tau applied the wrong
way, Self/Exchange maps swapped or mis-signed, a transposed evidence operand,
a zero-based count index, the mask on the wrong side, heads mixed up) are noted
per test.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import relation_oracle as O
from oracle.brute_mp import brute_head


def _rand_head(rng, T, d, scale=1.0):
    return tuple(rng.standard_normal((T, d)) * scale for _ in range(3))


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


# ---------------------------------------------------------------- maps ----

def test_maps_special_values_and_silu_minimum():
    """sigma(0)=1/2, SiLU(0)=0, both finite at +-1000, and SiLU's minimum is
    -W(1/e) = -0.27846... (the bounded negative tail the blog motivates; a map
    like u*sigmoid(-u) or a plain sigmoid fails this)."""
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    assert O.silu(np.array([0.0]))[0] == 0.0
    big = O.sigmoid(np.array([-1000.0, 1000.0]))
    assert big[0] == 0.0 and big[1] == 1.0
    s = O.silu(np.array([-1000.0, 1000.0]))
    assert s[0] == 0.0 and s[1] == 1000.0
    grid = np.linspace(-4, 2, 600001)
    vals = O.silu(grid)
    w = float(np.real(scipy.special.lambertw(1.0 / math.e)))
    assert abs(vals.min() + w) < 1e-10
    assert abs(grid[np.argmin(vals)] - (-1.0 - w)) < 2e-5
    x = np.linspace(-30, 30, 101)
    np.testing.assert_allclose(O.sigmoid(x) + O.sigmoid(-x), 1.0, rtol=0, atol=1e-15)


# ---------------------------------------------------------- P1 flow ------

@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_flow_is_row_stochastic_and_causal(lam):
    """Every row of F sums to 1 and F_ij = 0 above the diagonal (Eq. (3), (7))."""
    rng = np.random.default_rng(1)
    p1, p2, v = _rand_head(rng, 37, 8)
    _, F = O.relation_head(p1, p2, v, 0.7, lam, return_flow=True)
    np.testing.assert_allclose(F.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(F[np.triu_indices(37, k=1)] == 0.0)
    assert np.all(F >= 0.0)


# ---------------------------------------------------- P2 first token -----

def test_first_row_is_first_information_state():
    """The first token's history is empty, so F_11 = 1 and Y_1 = V_1 exactly
    (App. A.1.7), whatever P1, P2, tau, lambda."""
    rng = np.random.default_rng(2)
    for lam in (0.0, 0.5, -1.0):
        p1, p2, v = _rand_head(rng, 9, 5, scale=3.0)
        Y = O.relation_head(p1, p2, v, 0.3, lam)
        assert np.array_equal(Y[0], v[0])
        assert np.array_equal(O.flash_scan_head(p1, p2, v, 0.3, lam)[0], v[0])


# -------------------------------------------------- P3 T = 2 closed form --

@pytest.mark.parametrize("d", [1, 3, 8])
@pytest.mark.parametrize("tau", [0.5, 1.0, 2.0])
@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_two_token_closed_form(d, tau, lam):
    """Two tokens, derived by hand from Eq. (1)-(3):
        Y_1 = V_1,
        Y_2 = sigma(S_2 - E_21 + lam log 2) V_2 + sigma(E_21 - lam log 2 - S_2) V_1,
    with S_2 = sigma(p1_2.p2_2 / (tau sqrt d)) and E_21 = SiLU(p1_2.p2_1 / sqrt d).
    Catches a dropped 1/sqrt(d), tau multiplied instead of divided, a
    transposed evidence operand (p1_1.p2_2 in place of p1_2.p2_1), a zero-based
    count index (log 1 = 0) and swapped Self/Exchange maps."""
    rng = np.random.default_rng(100 + d)
    for _ in range(5):
        p1, p2, v = _rand_head(rng, 2, d, scale=1.5)
        Y = O.relation_head(p1, p2, v, tau, lam)
        s2 = _sig(float(np.dot(p1[1], p2[1])) / (tau * math.sqrt(d)))
        u21 = float(np.dot(p1[1], p2[0])) / math.sqrt(d)
        e21 = u21 * _sig(u21)
        w_self = _sig(s2 - e21 + lam * math.log(2.0))
        w_hist = _sig(e21 - lam * math.log(2.0) - s2)
        expect2 = w_self * v[1] + w_hist * v[0]
        np.testing.assert_allclose(Y[0], v[0], rtol=0, atol=0)
        np.testing.assert_allclose(Y[1], expect2, rtol=1e-14, atol=1e-14)


# -------------------------------------------- P5 zero evidence closed form --

@pytest.mark.parametrize("lam", [0.0, 0.5, 1.3])
def test_zero_evidence_prefix_form(lam):
    """With P2 = 0 every U is 0, so S_i = 1/2 (any tau) and E_ij = 0:
        Y_i = (e^{1/2} V_i + i^{-lam} sum_{j<i} V_j) / (e^{1/2} + i^{-lam} (i - 1)),
    i one-based. Catches an off-by-one count index, the diagonal counted in the
    history, and a wrong Self map value at zero."""
    rng = np.random.default_rng(5)
    T, d = 50, 6
    p1 = rng.standard_normal((T, d))
    p2 = np.zeros((T, d))
    v = rng.standard_normal((T, d))
    Y = O.relation_head(p1, p2, v, 0.37, lam)
    i = np.arange(1, T + 1, dtype=np.float64)[:, None]
    prefix = np.vstack([np.zeros((1, d)), np.cumsum(v, axis=0)[:-1]])
    eh = math.exp(0.5)
    expect = (eh * v + i ** (-lam) * prefix) / (eh + i ** (-lam) * (i - 1))
    np.testing.assert_allclose(Y, expect, rtol=1e-13, atol=1e-13)


# ------------------------------------------- textbook special case --------

def test_large_evidence_reduces_to_strictly_causal_softmax_attention():
    """When every U_ij is >= 20, SiLU(U) = U to within 40 e^-20 and the Exchange
    mass g_i = sigma(A_i - S_i) is 1 to within e^-18, so for i >= 2 the operator is
    textbook softmax attention over the strict history j < i with Q = P1, K = P2
    (scipy's softmax). Catches a transposed operand, the mask on the wrong side,
    a missing 1/sqrt(d_h) and the diagonal leaking into the history."""
    rng = np.random.default_rng(7)
    T, d = 24, 16
    base = np.full(d, math.sqrt(30.0 / math.sqrt(d)))    # U ~ 30 before noise
    p1 = base + 0.35 * rng.standard_normal((T, d))
    p2 = base + 0.35 * rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    U = p1 @ p2.T / math.sqrt(d)
    assert U.min() > 20.0 and U.max() < 45.0
    Y = O.relation_head(p1, p2, v, 1.0, 0.0)
    for r in range(1, T):
        w = scipy.special.softmax(U[r, :r])
        np.testing.assert_allclose(Y[r], w @ v[:r], rtol=0, atol=1e-6)


# ------------------------------------------------ P4 brute force ----------

@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_arbitrary_precision(seed):
    rng = np.random.default_rng(200 + seed)
    T = int(rng.integers(1, 9))
    d = int(rng.integers(1, 5))
    tau = [0.5, 1.0, 2.0][seed % 3]
    lam = [0.0, 0.5][seed % 2]
    p1, p2, v = _rand_head(rng, T, d, scale=1.7)
    Y = O.relation_head(p1, p2, v, tau, lam)
    ref = brute_head(p1.tolist(), p2.tolist(), v.tolist(), tau, lam)
    ref = np.array([[float(x) for x in row] for row in ref])
    np.testing.assert_allclose(Y, ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------ P6 factorization --------

@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_self_exchange_factorization(lam):
    """F_ii = sigma(S_i - A_i), sum_{j<i} F_ij = g_i, F_ij = g_i pi_ij,
    Y_i = (1 - g_i) V_i + g_i Ibar_i = V_i + g_i (Ibar_i - V_i)
    (Eq. (6)-(9), App. A.1.3-A.1.6, and the blog's later Delta form)."""
    rng = np.random.default_rng(9)
    T, d = 29, 7
    p1, p2, v = _rand_head(rng, T, d, scale=1.4)
    Y, F = O.relation_head(p1, p2, v, 0.8, lam, return_flow=True)
    fz = O.factorized_head(p1, p2, v, 0.8, lam)
    idx = np.arange(T)
    np.testing.assert_allclose(F[idx, idx], fz["F_self"], rtol=0, atol=1e-14)
    g_from_F = np.array([F[r, :r].sum() for r in range(T)])
    np.testing.assert_allclose(g_from_F, fz["g"], rtol=0, atol=1e-14)
    for r in range(1, T):
        np.testing.assert_allclose(F[r, :r], fz["g"][r] * fz["pi"][r, :r], rtol=0, atol=1e-14)
        delta = fz["Ibar"][r] - v[r]
        np.testing.assert_allclose(Y[r], v[r] + fz["g"][r] * delta, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Y, fz["Y"], rtol=0, atol=1e-13)
    assert fz["g"][0] == 0.0 and fz["F_self"][0] == 1.0


def test_count_correction_cancels_inside_history():
    """R_ij - R_ik = E_ij - E_ik, so pi is the same for every lambda (Eq. (11),
    App. A.1.5), while g moves with lambda (Eq. (10))."""
    rng = np.random.default_rng(10)
    p1, p2, v = _rand_head(rng, 20, 5)
    a = O.factorized_head(p1, p2, v, 1.0, 0.0)
    b = O.factorized_head(p1, p2, v, 1.0, 0.9)
    np.testing.assert_allclose(a["pi"], b["pi"], rtol=0, atol=1e-15)
    i = np.arange(1, 21)
    np.testing.assert_allclose(a["A"][1:] - b["A"][1:], 0.9 * np.log(i[1:]), rtol=0, atol=1e-12)
    assert np.all(b["g"][2:] < a["g"][2:])


# --------------------------------------------- P7 linearity / convexity ---

def test_linear_and_convex_in_information():
    rng = np.random.default_rng(11)
    T, d = 31, 6
    p1, p2, v = _rand_head(rng, T, d)
    w = rng.standard_normal((T, d))
    Yv = O.relation_head(p1, p2, v, 1.0)
    Yw = O.relation_head(p1, p2, w, 1.0)
    Yc = O.relation_head(p1, p2, 2.5 * v - 0.75 * w, 1.0)
    np.testing.assert_allclose(Yc, 2.5 * Yv - 0.75 * Yw, rtol=0, atol=1e-13)
    const = np.tile(rng.standard_normal(d), (T, 1))
    np.testing.assert_allclose(O.relation_head(p1, p2, const, 1.0), const, rtol=0, atol=1e-14)
    assert np.all(np.abs(Yv) <= np.abs(v).max(axis=0) + 1e-14)


# ----------------------------------------------------- P8 causality -------

def test_future_rows_do_not_change_the_past():
    rng = np.random.default_rng(12)
    T, d, cut = 40, 8, 17
    p1, p2, v = _rand_head(rng, T, d)
    Y = O.relation_head(p1, p2, v, 1.0, 0.5)
    q1, q2, qv = p1.copy(), p2.copy(), v.copy()
    q1[cut + 1:] += 5.0
    q2[cut + 1:] *= -3.0
    qv[cut + 1:] = 1e6
    Yq = O.relation_head(q1, q2, qv, 1.0, 0.5)
    np.testing.assert_allclose(Yq[:cut + 1], Y[:cut + 1], rtol=0, atol=1e-15)
    assert not np.allclose(Yq[cut + 1:], Y[cut + 1:])


# ------------------------------------------------- P9 exact cache ---------

def test_decode_is_last_row_of_forward():
    """Relation Cache {P2_1:t, I~_1:t} is exact (Eq. (18), App. A.5.2): one
    decode step equals the last forward row on [cache; new token]; cache rows
    past the length (NaN here) are never read."""
    rng = np.random.default_rng(13)
    B, H, d, Lcap = 3, 2, 5, 12
    lens = np.array([0, 7, 12])
    cP2 = np.full((B, H, Lcap, d), np.nan)
    cV = np.full((B, H, Lcap, d), np.nan)
    for b in range(B):
        cP2[b, :, :lens[b]] = rng.standard_normal((H, lens[b], d))
        cV[b, :, :lens[b]] = rng.standard_normal((H, lens[b], d))
    p1, p2, v = (rng.standard_normal((B, H, d)) for _ in range(3))
    tau = np.array([0.5, 2.0])
    for lam in (0.0, 0.5):
        y = O.relation_decode(p1, p2, v, cP2, cV, lens, tau, lam)
        assert np.all(np.isfinite(y))
        for b in range(B):
            L = lens[b]
            for h in range(H):
                P1s = np.vstack([rng.standard_normal((L, d)), p1[b, h][None]])
                P2s = np.vstack([cP2[b, h, :L], p2[b, h][None]])
                Vs = np.vstack([cV[b, h, :L], v[b, h][None]])
                Yf = O.relation_head(P1s, P2s, Vs, tau[h], lam)
                np.testing.assert_allclose(y[b, h], Yf[L], rtol=0, atol=1e-13)
    np.testing.assert_array_equal(y[0], v[0])


# --------------------------------------------- P10 head independence ------

def test_heads_are_independent():
    rng = np.random.default_rng(14)
    B, H, T, d = 2, 4, 11, 3
    P1, P2, V = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    tau = np.array([0.5, 1.0, 1.5, 2.0])
    Y = O.relation_fwd(P1, P2, V, tau, 0.2)
    perm = np.array([2, 0, 3, 1])
    Yp = O.relation_fwd(P1[:, perm], P2[:, perm], V[:, perm], tau[perm], 0.2)
    np.testing.assert_array_equal(Yp, Y[:, perm])
    np.testing.assert_array_equal(O.relation_fwd(P1[1:], P2[1:], V[1:], tau, 0.2), Y[1:])


# ------------------------------------------ P11 tiled scan == full ---------

@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_flash_scan_equals_materialized(lam):
    """FlashRelation is exact (App. A.3.5): the tiled (m, l, z) route with
    random tile boundaries equals the materialized definition."""
    rng = np.random.default_rng(15)
    T, d = 45, 6
    p1, p2, v = _rand_head(rng, T, d, scale=1.8)
    Y = O.relation_head(p1, p2, v, 0.6, lam)
    for _ in range(4):
        cuts = np.sort(rng.choice(np.arange(1, T), size=int(rng.integers(1, 10)), replace=False))
        bounds = [0] + cuts.tolist() + [T]
        Ys = O.flash_scan_head(p1, p2, v, 0.6, lam, bounds)
        np.testing.assert_allclose(Ys, Y, rtol=0, atol=1e-12)


def test_rows_route_matches_materialized():
    """The per-row route used for sampled checks at large T agrees with the
    materialized head at every row."""
    rng = np.random.default_rng(16)
    p1, p2, v = _rand_head(rng, 33, 4)
    Y = O.relation_head(p1, p2, v, 1.3, 0.5)
    rows = list(range(33))
    np.testing.assert_allclose(O.relation_rows(p1, p2, v, 1.3, 0.5, rows), Y, rtol=0, atol=1e-13)

"""Pins for the Linear Relation oracle (``oracle/linear_oracle.py``), fixed by
the pages and by algebra rather than by retyping the recurrence:
  * the unrolled state and read of [paper] App. A.4.4-A.4.5 (a second route,
    no recurrent state) agree with the recurrence;
  * a hand-derived 3-token, d_h = 1 example;
  * strict historical support (App. A.4.3): Y_t = I_t + (terms of tokens < t),
    and nothing at t changes earlier outputs;
  * T = 1 gives Y = I; vanishing retention forgets the history;
  * linearity in I; invariance of Y under a common rotation of P1 and P2
    when the retention is the same on every channel.
Mistakes these catch: p^1 / p^2 swapped, write before read, the decay of
step t not applied to the read of step t, S_t dropped from read or write,
unnormalised coordinates, tau misplaced.
"""
import math

import numpy as np
import pytest

from oracle import linear_oracle as LO


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def _head(rng, T, d, lo=0.3):
    p1, p2, I = (rng.standard_normal((T, d)) for _ in range(3))
    alpha = rng.uniform(lo, 1.0, (T, d))
    return p1, p2, I, alpha


@pytest.mark.parametrize("T,d,tau,seed", [(1, 3, 1.0, 0), (5, 2, 0.7, 1), (9, 4, 2.0, 2), (12, 6, 1.3, 3)])
def test_recurrence_equals_unrolled_form(T, d, tau, seed):
    rng = np.random.default_rng(seed)
    p1, p2, I, alpha = _head(rng, T, d)
    np.testing.assert_allclose(LO.linear_relation_head(p1, p2, I, alpha, tau),
                               LO.linear_relation_unrolled(p1, p2, I, alpha, tau), rtol=1e-12, atol=1e-12)


def test_final_state_equals_unrolled_state():
    """C_T = sum_j (prod_{u=j+1..T} D_u) S_j p^2_j I_j^T ([paper] App. A.4.4)."""
    rng = np.random.default_rng(4)
    T, d = 7, 3
    p1, p2, I, alpha = _head(rng, T, d)
    _, C = LO.linear_relation_head(p1, p2, I, alpha, 0.9, return_state=True)
    S = LO.self_relation(p1, p2, 0.9)
    k = p2 / np.linalg.norm(p2, axis=1, keepdims=True)
    want = np.zeros((d, d))
    for j in range(T):
        want += np.prod(alpha[j + 1:], axis=0)[:, None] * S[j] * np.outer(k[j], I[j])
    np.testing.assert_allclose(C, want, rtol=1e-12, atol=1e-13)


def test_hand_derived_three_tokens():
    """d_h = 1, tau = 1: p1 = (1, 2, -1), p2 = (1, 1, 3), I = (1, 2, 3),
    alpha = (1, 1/2, 1). Normalised coordinates are signs: p^1 = (1, 1, -1),
    p^2 = (1, 1, 1); S = (s(1), s(2), s(-3)).
      Y_1 = 1
      Y_2 = 2 + s(2) * (1/2) * s(1) * 1                 (history decayed by alpha_2)
      Y_3 = 3 - s(-3) * ((1/2) s(1) * 1 + s(2) * 2)    (token 1 decayed by alpha_2 alpha_3)"""
    p1 = np.array([[1.0], [2.0], [-1.0]])
    p2 = np.array([[1.0], [1.0], [3.0]])
    I = np.array([[1.0], [2.0], [3.0]])
    alpha = np.array([[1.0], [0.5], [1.0]])
    Y = LO.linear_relation_head(p1, p2, I, alpha, 1.0)[:, 0]
    want = [1.0, 2.0 + 0.5 * sig(2) * sig(1), 3.0 - sig(-3) * (0.5 * sig(1) + 2.0 * sig(2))]
    np.testing.assert_allclose(Y, want, rtol=1e-14)


def test_strict_historical_support():
    rng = np.random.default_rng(5)
    T, d, t = 10, 4, 6
    p1, p2, I, alpha = _head(rng, T, d)
    Y = LO.linear_relation_head(p1, p2, I, alpha, 1.1)
    I2 = I.copy()
    I2[t] += 0.37
    Y2 = LO.linear_relation_head(p1, p2, I2, alpha, 1.1)
    np.testing.assert_array_equal(Y2[:t], Y[:t])
    np.testing.assert_allclose(Y2[t] - Y[t], 0.37, rtol=0, atol=1e-14)
    for arr in (p1, p2, alpha):
        a2 = arr.copy()
        a2[t] *= 0.5
        args = [p1, p2, I, alpha]
        args[[id(x) for x in args].index(id(arr))] = a2
        np.testing.assert_array_equal(LO.linear_relation_head(*args, 1.1)[:t], Y[:t])


def test_single_token_and_vanishing_retention():
    rng = np.random.default_rng(6)
    p1, p2, I, alpha = _head(rng, 1, 5)
    np.testing.assert_array_equal(LO.linear_relation_head(p1, p2, I, alpha, 1.0), I)
    p1, p2, I, _ = _head(rng, 8, 5)
    Y = LO.linear_relation_head(p1, p2, I, np.full((8, 5), 1e-13), 1.0)
    np.testing.assert_allclose(Y, I, rtol=0, atol=1e-11)


def test_linear_in_information_and_rotation_invariant_with_uniform_retention():
    rng = np.random.default_rng(7)
    T, d = 9, 5
    p1, p2, I, _ = _head(rng, T, d)
    alpha = np.repeat(rng.uniform(0.4, 1.0, (T, 1)), d, axis=1)      # same on every channel
    J = rng.standard_normal((T, d))
    f = lambda x, a=p1, b=p2: LO.linear_relation_head(a, b, x, alpha, 0.8)
    np.testing.assert_allclose(f(2.0 * I - 3.0 * J), 2.0 * f(I) - 3.0 * f(J), rtol=1e-12, atol=1e-12)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    np.testing.assert_allclose(f(I, p1 @ Q, p2 @ Q), f(I), rtol=1e-12, atol=1e-12)


def test_multihead_is_per_head():
    rng = np.random.default_rng(8)
    B, H, T, d = 2, 3, 5, 4
    P1, P2, I = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    A = rng.uniform(0.5, 1.0, (B, H, T, d))
    tau = np.array([0.6, 1.0, 1.9])
    Y, C = LO.linear_relation_fwd(P1, P2, I, A, tau, return_state=True)
    for b in range(B):
        for h in range(H):
            y, c = LO.linear_relation_head(P1[b, h], P2[b, h], I[b, h], A[b, h], tau[h], True)
            np.testing.assert_array_equal(Y[b, h], y)
            np.testing.assert_array_equal(C[b, h], c)


def test_self_relation_scale_and_two_tokens_at_d4():
    """Eq. (15): S = sigmoid(p1 . p2 / (tau sqrt(d_h))). With d_h = 4, tau = 2
    and p1 = p2 = (1, 1, 1, 1): S = sigmoid(4 / (2 * 2)) = sigmoid(1). Two
    tokens: Y_2 = I_2 + S_2 S_1 alpha_2 (p^2_1 . p^1_2) I_1 when alpha_2 is
    uniform over channels."""
    p = np.ones((1, 4))
    assert LO.self_relation(p, p, 2.0)[0] == pytest.approx(sig(1.0), rel=1e-15)
    p1 = np.array([[1.0, 1.0, 1.0, 1.0], [2.0, 0.0, 0.0, 0.0]])
    p2 = np.array([[0.0, 3.0, 0.0, 4.0], [1.0, 1.0, 1.0, 1.0]])
    I = np.array([[1.0, -2.0, 0.5, 3.0], [0.0, 1.0, 0.0, 1.0]])
    alpha = np.array([[1.0] * 4, [0.25] * 4])
    S1 = sig((0 + 3 + 0 + 4) / (2.0 * 2.0))                 # p1_1 . p2_1 = 7
    S2 = sig(2.0 / (2.0 * 2.0))                             # p1_2 . p2_2 = 2
    dot = np.dot(np.array([0.0, 0.6, 0.0, 0.8]), np.array([1.0, 0.0, 0.0, 0.0]))   # p^2_1 . p^1_2 = 0
    Y = LO.linear_relation_head(p1, p2, I, alpha, 2.0)
    np.testing.assert_allclose(Y[1], I[1] + S2 * S1 * 0.25 * dot * I[0], rtol=1e-14)
    # a non-orthogonal pair: p1_2 = (0, 1, 0, 1) -> p^1_2 = (0, 1, 0, 1)/sqrt2, p^2_1 . p^1_2 = 1.4/sqrt2
    p1[1] = [0.0, 1.0, 0.0, 1.0]
    S2 = sig(2.0 / (2.0 * 2.0))
    Y = LO.linear_relation_head(p1, p2, I, alpha, 2.0)
    np.testing.assert_allclose(Y[1], I[1] + S2 * S1 * 0.25 * (1.4 / math.sqrt(2.0)) * I[0], rtol=1e-14)

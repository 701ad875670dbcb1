"""Pins for the pre-step oracle (RoPE on P1/P2, Givens mixing of the
information heads), fixed by geometry rather than by retyping the oracle:
  * RoPE: position 0 is the identity; every row keeps its norm; a 2-D row
    rotates by exactly pos * base^0 radians (the textbook plane rotation,
    compared through complex multiplication); the product of two rotated rows
    depends only on the position difference; the two pair conventions agree
    up to a fixed permutation of the coordinates.
  * Givens: angle 0 is the identity, angle pi/2 swaps a pair with a sign, the
    pair's energy is preserved (the orthogonality stated in App. A.2.2),
    angles t then -t undo each other, every head sits in exactly one pair of
    each pairing and M_B wraps (H, 1).
  * The model forward is invariant to a common position offset (U depends on
    relative positions only once RoPE is applied to both sides).
Mistakes these catch: a sign flip in the rotation, sin/cos swapped, a
frequency exponent of -k/d instead of -2k/d, a pairing off by one, angle
index order.
"""
import math

import numpy as np
import pytest

from oracle import prestep_oracle as PO
from oracle import relation_oracle as RO


@pytest.mark.parametrize("mode", ["interleaved", "half"])
def test_rope_position_zero_is_identity_and_norms_are_kept(mode):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 16))
    np.testing.assert_allclose(PO.rope(x, np.zeros(7), 1e4, mode), x, rtol=0, atol=0)
    y = PO.rope(x, np.arange(7) * 97 + 3, 1e4, mode)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("mode", ["interleaved", "half"])
def test_rope_two_dims_is_a_plane_rotation_by_pos_radians(mode):
    """d = 2: one pair with frequency base^0 = 1, so position p turns the row
    by p radians: x + iy -> (x + iy) e^{ip}."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 2))
    pos = np.array([0, 1, 2, 10, 8191])
    y = PO.rope(x, pos, 1e4, mode)
    z = (x[:, 0] + 1j * x[:, 1]) * np.exp(1j * pos)
    np.testing.assert_allclose(y[:, 0], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[:, 1], z.imag, rtol=1e-12, atol=1e-12)


def test_rope_second_pair_frequency_is_base_to_minus_two_k_over_d():
    """d = 4, base 1e4: pair 1 turns by pos * 1e4^(-1/2) = pos / 100 radians."""
    x = np.array([[0.0, 0.0, 1.0, 0.0]])
    y = PO.rope(x, np.array([50]), 1e4, "interleaved")
    np.testing.assert_allclose(y[0, 2:], [math.cos(0.5), math.sin(0.5)], rtol=1e-13)
    xh = np.array([[0.0, 1.0, 0.0, 0.0]])           # half layout: pair 1 = (x1, x3)
    yh = PO.rope(xh, np.array([50]), 1e4, "half")
    np.testing.assert_allclose(yh[0, [1, 3]], [math.cos(0.5), math.sin(0.5)], rtol=1e-13)


@pytest.mark.parametrize("mode", ["interleaved", "half"])
def test_rope_scores_depend_on_relative_position_only(mode):
    rng = np.random.default_rng(2)
    p, q = rng.standard_normal((2, 1, 32))
    for i, j in [(0, 5), (100, 37), (4000, 4100)]:
        base_score = (PO.rope(p, [i], 1e4, mode) @ PO.rope(q, [j], 1e4, mode).T).item()
        for shift in (1, 17, 3000):
            s = (PO.rope(p, [i + shift], 1e4, mode) @ PO.rope(q, [j + shift], 1e4, mode).T).item()
            assert s == pytest.approx(base_score, rel=1e-9, abs=1e-9)


def test_rope_conventions_differ_by_a_coordinate_permutation():
    rng = np.random.default_rng(3)
    d = 12
    x = rng.standard_normal((6, d))
    perm = np.empty(d, dtype=int)                     # half-layout index -> interleaved index
    perm[: d // 2] = 2 * np.arange(d // 2)
    perm[d // 2:] = 2 * np.arange(d // 2) + 1
    xi = np.empty_like(x)
    xi[:, perm] = x
    pos = np.arange(6) * 13
    yi = PO.rope(xi, pos, 1e4, "interleaved")
    np.testing.assert_allclose(PO.rope(x, pos, 1e4, "half"), yi[:, perm], rtol=1e-13, atol=1e-13)


def test_pairings_cover_every_head_once_and_b_wraps():
    for H in (2, 4, 8):
        for p in ("A", "B"):
            heads = [h for pair in PO.head_pairs(H, p) for h in pair]
            assert sorted(heads) == list(range(H))
    assert PO.head_pairs(8, "A")[0] == (0, 1) and PO.head_pairs(8, "B")[-1] == (7, 0)
    assert PO.head_pairs(8, "B")[0] == (1, 2)
    with pytest.raises(ValueError):
        PO.head_pairs(3, "A")


@pytest.mark.parametrize("pairing", ["A", "B"])
def test_givens_identity_swap_energy_and_inverse(pairing):
    rng = np.random.default_rng(4)
    B, H, T, d = 2, 4, 5, 6
    I = rng.standard_normal((B, H, T, d))
    np.testing.assert_array_equal(PO.givens_mix(I, np.zeros(H // 2), pairing), I)
    sw = PO.givens_mix(I, np.full(H // 2, math.pi / 2), pairing)
    for a, b in PO.head_pairs(H, pairing):
        np.testing.assert_allclose(sw[:, a], -I[:, b], atol=1e-15)
        np.testing.assert_allclose(sw[:, b], I[:, a], atol=1e-15)
    th = rng.uniform(-3, 3, H // 2)
    mixed = PO.givens_mix(I, th, pairing)
    for a, b in PO.head_pairs(H, pairing):
        np.testing.assert_allclose(mixed[:, a] ** 2 + mixed[:, b] ** 2, I[:, a] ** 2 + I[:, b] ** 2, rtol=1e-12)
    np.testing.assert_allclose(PO.givens_mix(mixed, -th, pairing), I, rtol=1e-12, atol=1e-12)


def test_givens_angle_order_follows_the_pair_order():
    """Only pair k moves when only angle k is non-zero."""
    rng = np.random.default_rng(5)
    I = rng.standard_normal((1, 8, 3, 4))
    for k, (a, b) in enumerate(PO.head_pairs(8, "B")):
        th = np.zeros(4)
        th[k] = 0.7
        out = PO.givens_mix(I, th, "B")
        moved = [h for h in range(8) if not np.array_equal(out[:, h], I[:, h])]
        assert sorted(moved) == sorted([a, b])


@pytest.mark.parametrize("mode", ["interleaved", "half"])
def test_model_forward_is_invariant_to_a_common_position_offset(mode):
    rng = np.random.default_rng(6)
    B, H, T, d = 2, 2, 9, 8
    P1, P2, I = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    tau = np.array([0.7, 1.3])
    th = np.array([0.4])
    y0 = PO.relation_fwd_model(P1, P2, I, tau, 0.5, None, 1e4, mode, th, "A")
    y1 = PO.relation_fwd_model(P1, P2, I, tau, 0.5, np.array([5, 1234]), 1e4, mode, th, "A")
    np.testing.assert_allclose(y1, y0, rtol=1e-10, atol=1e-10)


def test_model_forward_without_presteps_is_the_operator():
    rng = np.random.default_rng(7)
    P1, P2, I = (rng.standard_normal((1, 2, 6, 4)) for _ in range(3))
    tau = np.array([1.0, 2.0])
    np.testing.assert_array_equal(PO.relation_fwd_model(P1, P2, I, tau, 0.5, mode="none"),
                                  RO.relation_fwd(P1, P2, I, tau, 0.5))

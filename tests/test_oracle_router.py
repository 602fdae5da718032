"""Pins of the router oracle (oracle/router.py) against what mathematics fixes:
exact rational logits, the two-expert logistic closed form, shift invariance,
overflow safety, the tie order, brute-force top-k, and planted mistakes."""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

from oracle import router as RT


def _f16(a):
    return np.asarray(a, dtype=np.float16)


def test_logits_exact_rational():
    """fp16 values are dyadic rationals: the exact dot product, rounded once,
    equals the float64 logits within float64 rounding of a short sum."""
    rng = np.random.default_rng(1)
    x, w = _f16(rng.standard_normal((3, 40))), _f16(rng.standard_normal((5, 40)) / 6)
    got = RT.router_logits(x, w)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], w[e]))
            assert abs(got[t, e] - float(exact)) <= 40 * 2.0 ** -52 * (abs(float(exact)) + 1)


def test_softmax_two_experts_is_logistic():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((50, 2)) * 4
    p = RT.softmax(z)
    assert np.allclose(p[:, 0], expit(z[:, 0] - z[:, 1]), rtol=1e-13, atol=1e-15)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_softmax_uniform_and_shift_invariance():
    assert np.array_equal(RT.softmax(np.zeros((2, 8))), np.full((2, 8), 1 / 8))
    rng = np.random.default_rng(3)
    z = rng.standard_normal((10, 16))
    for c in [-300.0, 7.5, 1e4]:
        assert np.allclose(RT.softmax(z + c), RT.softmax(z), rtol=1e-9, atol=1e-15)


def test_softmax_no_overflow():
    z = np.array([[1e4, 1e4 - 1.0, -1e4]])
    p = RT.softmax(z)
    assert np.isfinite(p).all()
    assert p[0, 0] == pytest.approx(expit(1.0), rel=1e-13)
    assert p[0, 2] == 0.0


def test_topk_ties_and_order():
    s = np.array([[0.1, 0.3, 0.3, 0.05, 0.3, 0.0]])
    ids, vals = RT.topk(s, 4)
    assert ids.tolist() == [[1, 2, 4, 0]]          # equal scores: lower index first
    assert vals.tolist() == [[0.3, 0.3, 0.3, 0.1]]
    ids, vals = RT.topk(s, 0)
    assert ids.shape == (1, 0)
    ids, _ = RT.topk(s, 6)
    assert sorted(ids[0].tolist()) == list(range(6))
    with pytest.raises(ValueError):
        RT.topk(s, 7)


def test_topk_brute_force():
    """Every chosen score >= every unchosen one; decreasing order; the chosen
    set is the best k-subset by score sum (enumerated)."""
    from itertools import combinations
    rng = np.random.default_rng(4)
    s = rng.random((30, 7))
    ids, vals = RT.topk(s, 3)
    for t in range(30):
        chosen = set(ids[t].tolist())
        rest = [s[t, e] for e in range(7) if e not in chosen]
        assert min(vals[t]) >= max(rest)
        assert list(vals[t]) == sorted(vals[t], reverse=True)
        best = max(combinations(range(7), 3), key=lambda c: sum(s[t, list(c)]))
        assert chosen == set(best)


def test_route_uniform_when_gate_is_zero():
    x = _f16(np.random.default_rng(5).standard_normal((4, 64)))
    ids, vals, p = RT.route(x, np.zeros((6, 64), np.float16), 2)
    assert ids.tolist() == [[0, 1]] * 4
    assert np.array_equal(vals, np.full((4, 2), 1 / 6))


def test_planted_mistakes_fail():
    """Mistakes a router could make, planted here, break the pins above."""
    rng = np.random.default_rng(6)
    x = _f16(rng.standard_normal((8, 8)))
    w = _f16(rng.standard_normal((8, 8)))
    good = RT.router_logits(x, w)
    assert not np.allclose(x.astype(np.float64) @ w.astype(np.float64), good)   # W not transposed
    z = good
    wrong_axis = np.exp(z - z.max(axis=0)) / np.exp(z - z.max(axis=0)).sum(axis=0)
    assert not np.allclose(wrong_axis.sum(axis=1), 1.0)                           # softmax over tokens
    no_norm = np.exp(z - z.max(axis=1, keepdims=True))
    assert not np.allclose(no_norm.sum(axis=1), 1.0)                              # no normalisation
    ids, _ = RT.topk(RT.softmax(z), 3)
    asc = np.argsort(RT.softmax(z), axis=1, kind="stable")[:, :3]                 # smallest instead
    assert not np.array_equal(ids, asc)

"""Pins of the row-softmax oracle (oracle/softmax.py) to values fixed by the
mathematics: closed forms, a 50-digit decimal brute force in the probability
form, shift invariance, the online normaliser recurrence, and a pure-Python
top-k.  CPU only."""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import softmax as osm

getcontext().prec = 50


def brute_softmax(row):
    """p_j = 1 / sum_k exp(x_k - x_j), lse = x_0 + ln sum_k exp(x_k - x_0),
    in decimal arithmetic; no maximum is subtracted."""
    xs = [Decimal(float(v)) for v in row]
    p = [Decimal(1) / sum((xk - xj).exp() for xk in xs) for xj in xs]
    lse = xs[0] + sum((xk - xs[0]).exp() for xk in xs).ln()
    return np.array([float(v) for v in p]), float(lse)


def test_constant_row_is_uniform():
    y, lse = osm.softmax(np.full((2, 7), 3.25))
    assert np.all(y == 1.0 / 7)
    assert np.allclose(lse, 3.25 + math.log(7), rtol=0, atol=1e-15)


@pytest.mark.parametrize("a,b", [(0.0, 0.0), (1.0, -2.0), (-30.0, 5.5), (700.0, 699.0)])
def test_two_values_give_the_logistic(a, b):
    y, lse = osm.softmax(np.array([[a, b]]))
    assert abs(y[0, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
    assert abs(y[0, 0] + y[0, 1] - 1.0) < 1e-15
    assert abs(lse[0] - (max(a, b) + math.log1p(math.exp(-abs(a - b))))) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_matches_decimal_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3, 1 + seed * 3)) * (1 + 10 * seed)
    y, lse = osm.softmax(x)
    for r in range(x.shape[0]):
        p, l_ref = brute_softmax(x[r])
        assert np.allclose(y[r], p, rtol=1e-13, atol=1e-300)
        assert abs(lse[r] - l_ref) <= 1e-13 * max(1.0, abs(l_ref))


def test_shift_invariance_and_large_values():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 50))
    y0, l0 = osm.softmax(x)
    y1, l1 = osm.softmax(x * 1 + 1000.0)
    assert np.allclose(y0, y1, rtol=1e-12, atol=0)
    assert np.allclose(l1 - l0, 1000.0, rtol=0, atol=1e-10)
    y2, l2 = osm.softmax(x * 1000.0)  # exp of unshifted values would overflow
    assert np.all(np.isfinite(y2)) and np.allclose(y2.sum(-1), 1.0, atol=1e-14)


def test_online_normaliser_recurrence_gives_the_same_result():
    # One pass per row: m_j = max(m_{j-1}, x_j), d_j = d_{j-1} e^{m_{j-1}-m_j}
    # + e^{x_j - m_j} (the notebook's running maximum and denominator), then
    # y_j = e^{x_j - m_n} / d_n.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 200)) * 20
    y, lse = osm.softmax(x)
    for r in range(x.shape[0]):
        m, d = -math.inf, 0.0
        for v in x[r]:
            mn = max(m, v)
            d = d * math.exp(m - mn) + math.exp(v - mn)
            m = mn
        assert abs(m + math.log(d) - lse[r]) < 1e-12
        assert np.allclose(np.exp(x[r] - m) / d, y[r], rtol=1e-12, atol=0)


def brute_topk(row, k):
    return [j for _, j in sorted(((-float(v), j) for j, v in enumerate(row)))[:k]]


@pytest.mark.parametrize("k", [1, 3, 8])
def test_topk_matches_sorting_by_hand(k):
    rng = np.random.default_rng(20 + k)
    x = np.round(rng.standard_normal((5, 12)) * 2) / 2  # ties on purpose
    idx = osm.topk(x, k)
    probs, idx2, lse = osm.softmax_topk(x, k)
    y, _ = osm.softmax(x)
    for r in range(x.shape[0]):
        assert list(idx[r]) == brute_topk(x[r], k)
        assert np.array_equal(idx2[r], idx[r])
        assert np.array_equal(probs[r], y[r, idx[r]])
    assert np.all(np.diff(probs, axis=-1) <= 0)


def test_topk_ties_take_the_lower_index_first():
    x = np.array([[1.0, 5.0, 5.0, 2.0, 5.0]])
    assert list(osm.topk(x, 4)[0]) == [1, 2, 4, 3]
    with pytest.raises(ValueError):
        osm.topk(x, 6)

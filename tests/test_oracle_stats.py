"""Pins of the oracle's skew statistics of S (DODOCO summary, "metrics").

Independent checks: closed forms (uniform loads -> Gini 0 and max/mean 1;
one-hot -> Gini (n-1)/n; two-level loads), exact Python-integer brute force,
the sorted-rank formula of the Gini coefficient, and the golden example.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from helpers import load_golden


def test_uniform_counts():
    s = oracle.stats(np.full(64, 17, np.int32), 8)
    assert s["expert_gini"] == 0.0 and s["rank_gini"] == 0.0
    assert s["expert_max_over_mean"] == 1.0 and s["rank_max_over_mean"] == 1.0
    assert s["total"] == 64 * 17


@pytest.mark.parametrize("n", [2, 5, 16, 256])
def test_one_hot_gini(n):
    v = np.zeros(n, np.int64)
    v[n // 3] = 1234
    assert oracle.gini(v) == pytest.approx((n - 1) / n, rel=1e-15)


def test_two_level_closed_form():
    # m of n entries equal a, the rest b: Gini = m (n-m) |a-b| / (n (m a + (n-m) b))
    n, m, a, b = 40, 7, 90, 3
    v = np.array([a] * m + [b] * (n - m))
    ref = m * (n - m) * abs(a - b) / (n * (m * a + (n - m) * b))
    assert oracle.gini(v) == pytest.approx(ref, rel=1e-15)


def test_gini_sorted_rank_formula():
    g = np.random.default_rng(0)
    for _ in range(20):
        v = g.integers(0, 1000, size=int(g.integers(1, 80)))
        s = np.sort(v)
        n = len(s)
        if s.sum() == 0:
            continue
        i = np.arange(1, n + 1)
        ref = Fraction(int(((2 * i - n - 1) * s).sum()), int(n * s.sum()))
        assert oracle.gini(v) == float(ref)


def test_stats_bruteforce_exact():
    g = np.random.default_rng(1)
    E, R = 48, 6
    c = g.integers(0, 500, size=E).astype(np.int32)
    s = oracle.stats(c, R)
    L = E // R
    loads = [int(c[r * L:(r + 1) * L].sum()) for r in range(R)]
    tot = int(c.sum())

    def gini_exact(v):
        return float(Fraction(sum(abs(a - b) for a in v for b in v), 2 * len(v) * sum(v)))

    assert s["expert_gini"] == gini_exact([int(a) for a in c])
    assert s["rank_gini"] == gini_exact(loads)
    assert s["expert_max_over_mean"] == float(Fraction(int(c.max()) * E, tot))
    assert s["rank_max_over_mean"] == float(Fraction(max(loads) * R, tot))
    assert (s["expert_max"], s["expert_min"], s["rank_max"], s["rank_min"]) == \
        (int(c.max()), int(c.min()), max(loads), min(loads))


def test_zero_total():
    s = oracle.stats(np.zeros(8, np.int32), 2)
    assert s["expert_gini"] == 0.0 and s["expert_max_over_mean"] == 0.0 and s["total"] == 0


def test_rank_view_invariant_to_expert_order_within_rank():
    # Per-rank Gini depends only on the row sums of S.
    g = np.random.default_rng(2)
    c = g.integers(0, 100, size=32).astype(np.int32)
    c2 = c.reshape(4, 8)[:, ::-1].ravel().copy()
    assert oracle.stats(c, 4)["rank_gini"] == oracle.stats(c2, 4)["rank_gini"]


def test_golden_tiny():
    g = load_golden("dispatch_waves_tiny.txt")
    s = oracle.stats(np.array(g["expert_counts"], np.int32), int(g["R"][0]))
    for key in ("expert_max_over_mean", "expert_gini", "rank_max_over_mean", "rank_gini"):
        assert s[key] == g[key][0], key

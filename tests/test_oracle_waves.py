"""Pins of the oracle's wave-count and link-tail models (irregular AllToAll
page): the page's worked NVLink 5.0 example, the calculus of T(W), brute force
over the divisors of L, and a multinomial simulation of the p95 link volume."""
import numpy as np
import pytest

import oracle
from helpers import load_golden


def test_page_example_w_star_about_18():
    g = load_golden("wave_model_nvlink5.txt")
    w = oracle.optimal_waves(g["M_bytes"][0], g["alpha_s"][0], g["beta_Bps"][0])
    assert abs(w - g["W_star_about"][0]) < 0.5
    # 16 MiB instead of 16 MB reads the same
    assert abs(oracle.optimal_waves(16 * 2**20, 1e-6, 50e9) - 18) < 0.5


@pytest.mark.parametrize("M,a,b", [(16e6, 1e-6, 50e9), (2e9, 2e-6, 153e9), (1e5, 5e-6, 10e9)])
def test_w_star_minimises_t(M, a, b):
    ws = np.linspace(0.05, 400, 400001)
    t = ws * a + M / b + M / (ws * b)
    w_grid = ws[np.argmin(t)]
    w = oracle.optimal_waves(M, a, b)
    assert abs(w_grid - w) <= 2e-3 * max(w, 1)
    assert oracle.wave_time(M, a, b, w) <= min(oracle.wave_time(M, a, b, w * f)
                                               for f in (0.9, 1.1))
    # T at the optimum: M/b + 2 sqrt(M a / b)
    assert abs(oracle.wave_time(M, a, b, w) - (M / b + 2 * np.sqrt(M * a / b))) <= 1e-12 * M / b


@pytest.mark.parametrize("L", [1, 8, 12, 18, 32, 64])
def test_plan_is_the_best_divisor(L):
    M, a, b = 16e6, 1e-6, 50e9
    divs = [w for w in range(1, L + 1) if L % w == 0]
    want = min(divs, key=lambda w: (w * a + M / b + M / (w * b), w))
    assert oracle.plan_waves(M, a, b, L) == want


def test_p95_formula_against_multinomial_simulation():
    g = np.random.default_rng(0)
    bytes_per_token = 1000.0
    for B, n in ((4096, 8), (16384, 32), (2048, 16)):  # B p >= 10
        loads = g.multinomial(B, np.full(n, 1.0 / n), size=20000).ravel() * bytes_per_token
        m_avg = B / n * bytes_per_token
        emp = np.percentile(loads, 95)
        assert abs(emp / oracle.link_p95(m_avg, B, n) - 1) < 0.02
    # small B p (= 2): the page warns that the normal estimate fails there and that
    # p95 reaches twice the mean and more
    loads = g.multinomial(32, np.full(16, 1 / 16), size=20000).ravel()
    emp = np.percentile(loads, 95)
    assert emp >= 2 * loads.mean()
    assert abs(emp / oracle.link_p95(2.0, 32, 16) - 1) > 0.02

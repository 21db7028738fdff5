"""Pins of the oracle's fitted symmetric Dirichlet alpha (DODOCO summary,
"metrics"; read as the maximum-likelihood alpha of a Dirichlet-multinomial):
recovery of a known alpha from simulated routings, the score at the estimate
evaluated with scipy's digamma (an independent route to the same derivative),
maximality against scipy's log-gamma likelihood, and the limits."""
import math

import numpy as np
import pytest
from scipy.special import digamma, gammaln

import oracle
import synth


def _counts(seed, E, N, alpha):
    g = np.random.default_rng(seed)
    p = g.dirichlet(np.full(E, alpha))
    return np.bincount(g.choice(E, size=N, p=p), minlength=E).astype(np.int32)


def _loglik(c, a):
    E, N = c.shape[0], c.sum()
    return gammaln(E * a) - gammaln(N + E * a) + np.sum(gammaln(c + a) - gammaln(a))


def _score(c, a):
    E, N = c.shape[0], c.sum()
    return np.sum(digamma(c + a) - digamma(a)) - E * (digamma(N + E * a) - digamma(E * a))


@pytest.mark.parametrize("E,N,alpha", [(256, 131072, 0.3), (64, 60000, 1.0), (64, 60000, 3.0),
                                       (128, 80000, 0.1)])
def test_recovers_known_alpha(E, N, alpha):
    # one routing draw estimates alpha from E samples of p (spread ~ alpha*sqrt(2/E));
    # the mean over 8 independent draws must land within 15%
    est = [oracle.dirichlet_alpha(_counts(seed, E, N, alpha)) for seed in range(8)]
    assert abs(np.mean(est) / alpha - 1) < 0.15, est


@pytest.mark.parametrize("seed,E,N,alpha", [(5, 256, 131072, 0.3), (6, 16, 5000, 2.0),
                                            (7, 8, 200, 0.5)])
def test_score_vanishes_and_likelihood_is_maximal(seed, E, N, alpha):
    c = _counts(seed, E, N, alpha)
    a = oracle.dirichlet_alpha(c)
    assert 0 < a < math.inf
    scale = np.sum(np.abs(digamma(c + a) - digamma(a))) + E * abs(digamma(N + E * a))
    assert abs(_score(c, a)) <= 1e-9 * scale
    for f in (0.98, 0.995, 1.005, 1.02):
        assert _loglik(c, a * f) < _loglik(c, a)


def test_limits():
    assert oracle.dirichlet_alpha(np.full(64, 100)) == math.inf       # perfectly even
    assert oracle.dirichlet_alpha(np.array([500] + [0] * 63)) == 0.0   # one expert takes all
    assert math.isnan(oracle.dirichlet_alpha(np.zeros(8, np.int32)))  # no picks
    assert math.isnan(oracle.dirichlet_alpha(np.array([7], np.int32)))  # one category
    # multinomial sampling with equal probabilities is at the no-overdispersion end
    g = np.random.default_rng(3)
    c = np.bincount(g.integers(0, 64, 100000), minlength=64).astype(np.int32)
    assert oracle.dirichlet_alpha(c) > 50


def test_permutation_invariant():
    c = _counts(8, 32, 4000, 0.7)
    g = np.random.default_rng(0)
    a = oracle.dirichlet_alpha(c)
    b = oracle.dirichlet_alpha(c[g.permutation(32)])
    assert abs(a - b) <= 1e-12 * a


def test_generator_alpha_and_routing_sharpening():
    """The dirichlet_waves generator draws p ~ Dirichlet(0.3) over E = 256: counts
    drawn straight from Multinomial(T k, p) fit alpha close to 0.3 (mean over six
    seeds within 15%). The workload's routed counts (top-8 of N(0,1) + ln p) fit
    a much smaller alpha (about 0.09): an expert whose ln p lies far below the
    8th largest is almost never lifted into the top 8 by unit noise, and the
    largest ones are picked by almost every token, so fewer experts receive
    picks and the counts are more uneven than p itself."""
    wl = synth.WORKLOADS["dirichlet_waves"]
    mult, routed = [], []
    for seed in range(6):
        p = np.exp(synth._dirichlet_log_bias(wl.E, 0.3, seed).astype(np.float64))
        p /= p.sum()
        c = np.random.default_rng(100 + seed).multinomial(wl.T * wl.k, p).astype(np.int32)
        idx, _ = oracle.route(synth.logits(wl.with_(seed=seed)), wl.k)
        ec, _ = oracle.counts(idx, wl.E, wl.R, wl.W)
        a_m, a_r = oracle.dirichlet_alpha(c), oracle.dirichlet_alpha(ec)
        mult.append(a_m)
        routed.append(a_r)
        assert a_r < 0.5 * a_m
        assert (ec > 0).sum() < (c > 0).sum()
    assert abs(np.mean(mult) - 0.3) < 0.15 * 0.3
    assert 0.05 < np.mean(routed) < 0.15

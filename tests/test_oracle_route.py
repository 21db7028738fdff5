"""Pins of the oracle's top-k gating (MoE systems survey, section 1.1, eq. (2)).

Independent checks: numpy's stable argsort (library routine), a brute-force
Python sort, scipy's softmax on the kept logits, closed forms (k=1, k=2,
all-equal logits) and the hand-worked golden example.
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle
from helpers import load_golden


def _logits(T, E, seed, ties=False):
    g = np.random.default_rng(seed)
    if ties:
        return g.integers(-2, 3, size=(T, E)).astype(np.float32)
    return g.standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("T,E,k,ties", [(64, 8, 2, False), (50, 64, 6, False), (40, 256, 8, False),
                                        (33, 16, 16, False), (64, 8, 3, True), (40, 128, 8, True),
                                        (7, 5, 1, True), (9, 1024, 32, False)])
def test_indices_match_stable_argsort(T, E, k, ties):
    l = _logits(T, E, seed=T * E + k, ties=ties)
    idx, _ = oracle.route(l, k)
    # descending value, ties -> lower id == stable ascending sort of -l
    ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref)


def test_indices_bruteforce_python_sort():
    l = _logits(30, 6, seed=3, ties=True)
    idx, _ = oracle.route(l, 4)
    for t in range(l.shape[0]):
        ref = sorted(range(6), key=lambda e: (-float(l[t, e]), e))[:4]
        assert list(idx[t]) == ref


def test_topk_set_maximises_sum_bruteforce():
    # The kept set is a k-subset with the largest logit sum (checked over all subsets).
    l = _logits(20, 7, seed=11)
    k = 3
    idx, _ = oracle.route(l, k)
    for t in range(20):
        best = max(sum(float(l[t, e]) for e in c) for c in itertools.combinations(range(7), k))
        assert abs(sum(float(l[t, e]) for e in idx[t]) - best) < 1e-6


def test_weights_equal_softmax_of_kept_logits():
    l = _logits(200, 64, seed=5)
    idx, w = oracle.route(l, 6)
    kept = np.take_along_axis(l.astype(np.float64), idx, axis=1)
    ref = scipy.special.softmax(kept, axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-14, atol=0)


def test_weights_closed_forms():
    l = _logits(100, 16, seed=9)
    idx, w = oracle.route(l, 1)
    assert np.all(w == 1.0)
    idx, w = oracle.route(l, 2)
    d = np.take_along_axis(l.astype(np.float64), idx, axis=1)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(d[:, 1] - d[:, 0])), rtol=1e-15)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=4.5e-16)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_all_equal_logits():
    l = np.full((4, 10), 0.25, np.float32)
    idx, w = oracle.route(l, 4)
    assert (idx == np.arange(4)).all()
    assert np.all(w == 0.25)


def test_signed_zero_is_a_tie():
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    idx, w = oracle.route(l, 2)
    assert idx.tolist() == [[0, 1], [0, 1]]
    assert np.all(w == 0.5)


def test_k_equals_E_is_full_order():
    l = _logits(10, 8, seed=1)
    idx, w = oracle.route(l, 8)
    np.testing.assert_array_equal(idx, np.argsort(-l, axis=1, kind="stable"))
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-15)


def test_golden_tiny():
    g = load_golden("dispatch_waves_tiny.txt")
    l = np.array(g["logits"], np.float32)
    idx, w = oracle.route(l, int(g["k"][0]))
    np.testing.assert_array_equal(idx, np.array(g["topk_idx"], np.int32))
    np.testing.assert_allclose(w, np.array(g["topk_w"]), rtol=1e-15)

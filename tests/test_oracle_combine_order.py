"""Pins of the oracle's completion-wave order for the per-wave combine
(irregular AllToAll page, "Wave-Scheduled pipelining"): a hand-worked example,
numpy's stable argsort of independently computed completion waves, the row
layout of the oracle's own dispatch (every row of a wave's tokens lies in that
wave or an earlier one, and the last in that wave), and the special cases W = 1
and no kept picks."""
import numpy as np
import pytest

import oracle
from helpers import load_golden


def _ints(v):
    return np.array(v, dtype=np.int32)


def test_hand_worked_example():
    g = load_golden("combine_order_tiny.txt")
    T, E, k, R, W = (int(g[key][0]) for key in ("T", "E", "k", "R", "W"))
    idx = _ints(g["topk_idx"]).reshape(T, k)
    two, order = oracle.combine_order(idx, E, R, W)
    np.testing.assert_array_equal(two, _ints(g["token_wave_offsets"]))
    np.testing.assert_array_equal(order, _ints(g["token_order"]))


def _completion_numpy(idx, E, R, W):
    """The last wave of each token's kept picks, vectorised (0 without one)."""
    L = E // R
    kept = (idx >= 0) & (idx < E)
    wave = (np.where(kept, idx, 0) % L) * W // L
    return np.where(kept, wave, 0).max(axis=1) if idx.shape[1] else np.zeros(len(idx), int)


CASES = [(1, 8, 2, 2, 2, 0.0), (37, 16, 4, 4, 2, 0.1), (200, 64, 6, 4, 8, 0.2),
         (513, 32, 8, 1, 32, 0.05), (100, 8, 8, 2, 4, 0.0), (64, 1024, 32, 8, 16, 0.3),
         (300, 12, 3, 3, 4, 0.5), (50, 4, 1, 1, 4, 1.0)]


@pytest.mark.parametrize("T,E,k,R,W,drop", CASES)
def test_stable_argsort_of_completion_waves(T, E, k, R, W, drop):
    g = np.random.default_rng(T * 31 + E)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx = np.where(g.random(idx.shape) < drop, g.choice([-1, E, -7], idx.shape), idx)
    idx = idx.astype(np.int32)
    two, order = oracle.combine_order(idx, E, R, W)
    c = _completion_numpy(idx, E, R, W)
    np.testing.assert_array_equal(order, np.argsort(c, kind="stable"))
    np.testing.assert_array_equal(two, np.concatenate([[0], np.cumsum(np.bincount(c, minlength=W))]))
    assert sorted(order.tolist()) == list(range(T))


@pytest.mark.parametrize("T,E,k,R,W,drop", CASES)
def test_against_the_dispatch_row_layout(T, E, k, R, W, drop):
    """Through the oracle's dispatch: wave w's rows are [wave_offsets[w],
    wave_offsets[w+1]); a token listed in wave w has all its rows before
    wave_offsets[w+1] and its last row at or after wave_offsets[w]."""
    g = np.random.default_rng(T * 7 + k)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx = np.where(g.random(idx.shape) < drop, -1, idx).astype(np.int32)
    x = np.zeros((T, 4), np.float32)
    d = oracle.dispatch(x, idx, E, R, W)
    wo, pos = d["wave_offsets"], d["pos"]
    two, order = oracle.combine_order(idx, E, R, W)
    for w in range(W):
        for t in order[two[w]:two[w + 1]]:
            rows = pos[t][pos[t] >= 0]
            if rows.size == 0:
                assert w == 0
                continue
            assert rows.max() < wo[w + 1] and rows.max() >= wo[w]


def test_one_wave_is_token_order():
    g = np.random.default_rng(5)
    idx = g.integers(0, 16, (40, 3)).astype(np.int32)
    two, order = oracle.combine_order(idx, 16, 4, 1)
    np.testing.assert_array_equal(two, [0, 40])
    np.testing.assert_array_equal(order, np.arange(40))


def test_no_kept_pick_is_wave_zero_and_empty_batch():
    idx = np.full((9, 2), -1, np.int32)
    two, order = oracle.combine_order(idx, 8, 2, 4)
    np.testing.assert_array_equal(two, [0, 9, 9, 9, 9])
    np.testing.assert_array_equal(order, np.arange(9))
    two, order = oracle.combine_order(np.zeros((0, 2), np.int32), 8, 2, 4)
    np.testing.assert_array_equal(two, [0, 0, 0, 0, 0])
    assert order.size == 0

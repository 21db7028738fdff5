"""Pins of the oracle's counts, offsets, positions and dispatch copy.

Independent checks: numpy.bincount / cumsum / stable argsort (library routines
that reach the same permutation a different way), the invariants the pages
state for the send-count matrix S (sum of S = T*k, row sums = per-rank send
counts), and the hand-worked golden example with W=2 waves.
"""
import numpy as np
import pytest

import oracle
from helpers import bucket_rank_of_expert, load_golden


def _idx(T, E, k, seed):
    l = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    return oracle.route(l, k)[0]


CASES = [(37, 8, 2, 4, 1), (200, 64, 6, 8, 1), (300, 256, 8, 32, 8), (64, 16, 2, 1, 1),
         (129, 128, 8, 16, 2), (90, 16, 4, 2, 4), (1, 8, 8, 2, 2), (55, 12, 3, 3, 2)]


@pytest.mark.parametrize("T,E,k,R,W", CASES)
def test_counts_are_bincount_and_S_sums(T, E, k, R, W):
    idx = _idx(T, E, k, seed=T + E)
    ec, rc = oracle.counts(idx, E, R, W)
    np.testing.assert_array_equal(ec, np.bincount(idx.ravel(), minlength=E))
    assert ec.sum() == T * k
    L = E // R
    S = ec.reshape(R, L)  # rows: destination rank, columns: local slot
    # per-rank Alltoallv send counts = row sums of S, split over waves
    np.testing.assert_array_equal(rc.reshape(W, R).sum(0), S.sum(1))
    # per-wave totals = sums over the wave's slot columns
    for w in range(W):
        cols = [s for s in range(L) if s * W // L == w]
        assert rc.reshape(W, R)[w].sum() == S[:, cols].sum()


@pytest.mark.parametrize("T,E,k,R,W", CASES)
def test_offsets_are_cumsum_in_bucket_order(T, E, k, R, W):
    idx = _idx(T, E, k, seed=2 * T + E)
    ec, rc = oracle.counts(idx, E, R, W)
    eo, ro, wo = oracle.offsets(ec, R, W)
    br = bucket_rank_of_expert(E, R, W)
    order = np.argsort(br)
    excl = np.concatenate([[0], np.cumsum(ec[order])[:-1]])
    ref = np.empty(E, np.int64)
    ref[order] = excl
    np.testing.assert_array_equal(eo, ref)
    np.testing.assert_array_equal(ro, np.concatenate([[0], np.cumsum(rc)[:-1]]))
    assert wo[0] == 0 and wo[-1] == T * k
    np.testing.assert_array_equal(wo[:-1], ro.reshape(W, R)[:, 0])


@pytest.mark.parametrize("T,E,k,R,W", CASES)
def test_positions_are_stable_argsort_of_bucket_key(T, E, k, R, W):
    idx = _idx(T, E, k, seed=3 * T + E)
    out = oracle.dispatch(np.zeros((T, 4), np.float32), idx, E, R, W)
    br = bucket_rank_of_expert(E, R, W)
    # row n of the send buffer holds pick order[n]; picks are numbered t*k + i
    order = np.argsort(br[idx.ravel()], kind="stable")
    ref_pos = np.empty(T * k, np.int64)
    ref_pos[order] = np.arange(T * k)
    np.testing.assert_array_equal(out["pos"].ravel(), ref_pos)
    np.testing.assert_array_equal(out["row_token"], order // k)
    # pos is a bijection onto [0, T*k)
    assert np.array_equal(np.sort(out["pos"].ravel()), np.arange(T * k))


def test_send_buffer_rows_are_token_rows():
    T, E, k, R, W = 77, 16, 4, 4, 2
    idx = _idx(T, E, k, seed=8)
    x = np.random.default_rng(1).standard_normal((T, 24)).astype(np.float32)
    out = oracle.dispatch(x, idx, E, R, W)
    np.testing.assert_array_equal(out["send_buf"], x[out["row_token"]])
    for t in range(T):
        for i in range(k):
            np.testing.assert_array_equal(out["send_buf"][out["pos"][t, i]], x[t])


def test_bf16_rows_copy_bitwise():
    T, E, k = 40, 8, 3
    idx = _idx(T, E, k, seed=4)
    x = np.random.default_rng(2).integers(0, 2**16, size=(T, 16), dtype=np.uint16)
    out = oracle.dispatch(x, idx, E, 2, 1)
    np.testing.assert_array_equal(out["send_buf"], x[out["row_token"]])


def test_dropped_picks():
    idx = np.array([[0, 5], [-1, 1], [1, 0]], np.int32)  # E=4: 5 and -1 are out of range
    out = oracle.dispatch(np.arange(12, dtype=np.float32).reshape(3, 4), idx, 4, 2, 1)
    assert out["expert_counts"].tolist() == [2, 2, 0, 0]
    assert out["pos"].tolist() == [[0, -1], [-1, 2], [3, 1]]
    assert out["row_token"].tolist() == [0, 2, 1, 2]
    assert out["nrows"] == 4


def test_empty_batch():
    idx = np.zeros((0, 2), np.int32)
    out = oracle.dispatch(np.zeros((0, 8), np.float32), idx, 8, 4, 1)
    assert out["expert_counts"].sum() == 0 and out["nrows"] == 0
    assert out["wave_offsets"].tolist() == [0, 0]


def test_golden_tiny():
    g = load_golden("dispatch_waves_tiny.txt")
    E, k, R, W = (int(g[n][0]) for n in ("E", "k", "R", "W"))
    idx = np.array(g["topk_idx"], np.int32)
    out = oracle.dispatch(np.eye(4, dtype=np.float32), idx, E, R, W)
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
                "wave_offsets", "pos", "row_token"):
        np.testing.assert_array_equal(out[key], np.array(g[key], np.int64), err_msg=key)

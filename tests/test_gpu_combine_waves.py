"""The combine of the wave schedule (irregular AllToAll page, wave-scheduled
pipelining: each wave's dispatch -> compute -> combine) through the C ABI:
moe_combine_order (tokens listed by the wave after which all their experts
have run) and moe_combine_waves (the combine of the tokens of a range of
completion waves).

Bars: the token tables bit-exact against the oracle's completion-wave order;
the combined tokens bit-identical to moe_combine on the same expert rows
(the same per-column fp32 chain) over every split of the waves, rows of
other waves untouched; and equal to the oracle's fp32 fma chain over the
oracle's own expert rows. Cases: several blocks of tokens with a ragged tail (and blocks of two
ranking batches), one wave, one slot per wave, 1024 waves, dropped picks,
tokens with no kept pick, empty and one-token batches, fp32 rows, the
dirichlet_waves size in full."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_parity import DEV, dev, host

pytestmark = pytest.mark.gpu


def _wl(T, H, E, k, R, W, dtype="bf16", routing="iid", seed=5):
    return synth.Workload("edge", T=T, H=H, dtype=dtype, E=E, k=k, R=R, W=W, routing=routing,
                          seed=seed)


CASES = {
    "dirichlet_shape": synth.WORKLOADS["dirichlet_waves"].with_(T=2500, H=256),
    "zipf_W4": synth.WORKLOADS["zipf"].with_(T=1500, H=128, W=4),
    "one_wave": _wl(700, 64, 16, 4, 4, 1),
    "slot_per_wave": _wl(1100, 64, 64, 6, 4, 16),
    "E1024_W32": _wl(3000, 64, 1024, 8, 8, 32),
    "k1": _wl(1025, 64, 32, 1, 2, 8),
    "ties": _wl(600, 64, 16, 4, 4, 2, routing="ties"),
    "f32": _wl(999, 32, 32, 3, 4, 2, dtype="f32"),
    "T1": _wl(1, 64, 16, 2, 2, 4),
    # 35 order blocks of 2048 tokens (two ranking batches a block), 1024 waves
    "W1024_two_batches_a_block": _wl(70000, 16, 1024, 1, 1, 1024),
}


def _inputs(wl, drop=0.0):
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx, w = oracle.route(logits, wl.k)
    if drop > 0:
        g = np.random.default_rng(wl.T + 1)
        idx = np.where(g.random(idx.shape) < drop, g.choice([-1, wl.E, -9], idx.shape), idx)
        idx = idx.astype(np.int32)
        # a few tokens with no kept pick at all
        idx[:: max(wl.T // 7, 1)] = -1
    return x, idx, w


def _shape(wl, T=None):
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    return moe.Shape(wl.T if T is None else T, wl.H, wl.E, wl.k, wl.R, wl.W, tdt)


def _run(wl, x, idx, w):
    """Index stage, scaled experts and the one-pass combine on the GPU."""
    shape = _shape(wl)
    xd, idd = dev(x), dev(idx)
    out = moe.dispatch(xd, idd, wl.E, wl.R, wl.W)
    eo = moe.expert_scale(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape)
    wd = dev(w.astype(np.float32))
    y = moe.combine(eo, wd, out["pos"], shape)
    return shape, out, eo, wd, y


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("drop", [0.0, 0.25])
@pytest.mark.parametrize("name", list(CASES))
def test_order_and_combine_by_wave(name, drop):
    wl = CASES[name]
    print(f"[combine waves] {name} drop={drop}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} "
          f"W={wl.W} {wl.dtype}", flush=True)
    x, idx, w = _inputs(wl, drop)
    shape, out, eo, wd, y_ref = _run(wl, x, idx, w)
    two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
    two_o, order_o = oracle.combine_order(idx, wl.E, wl.R, wl.W)
    np.testing.assert_array_equal(host(two), two_o)
    np.testing.assert_array_equal(host(order), order_o)

    # every wave on its own (16 of them beyond 32), rows of the other waves untouched
    waves = range(wl.W) if wl.W <= 32 else sorted({0, wl.W - 1, *np.random.default_rng(
        wl.W).choice(wl.W, 14, replace=False).tolist()})
    for w0 in waves:
        y = torch.empty_like(y_ref)
        y.view(torch.uint8).fill_(0xA5)
        moe.combine_waves(eo, wd, out["pos"], order, two, shape, w0, w0 + 1, y=y)
        mine = torch.zeros(wl.T, dtype=torch.bool, device=DEV)
        mine[order[int(two_o[w0]):int(two_o[w0 + 1])].long()] = True
        assert torch.equal(_bits(y[mine]), _bits(y_ref[mine])), w0
        assert bool((y.view(torch.uint8)[~mine] == 0xA5).all()), w0
    # all waves in one call, and an uneven split in two calls
    y = torch.empty_like(y_ref)
    moe.combine_waves(eo, wd, out["pos"], order, two, shape, 0, wl.W, y=y)
    assert torch.equal(_bits(y), _bits(y_ref))
    cut = (wl.W * 2) // 3
    y.view(torch.uint8).fill_(0x5A)
    moe.combine_waves(eo, wd, out["pos"], order, two, shape, cut, wl.W, y=y)
    moe.combine_waves(eo, wd, out["pos"], order, two, shape, 0, cut, y=y)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    # and the oracle's fp32 chain over the oracle's rows
    ref = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
    eo_o = oracle.expert_scale(ref["send_buf"], ref["expert_offsets"], ref["expert_counts"])
    y_o = oracle.combine_f32fma(eo_o, w.astype(np.float32), ref["pos"], wl.T)
    np.testing.assert_array_equal(host(y), y_o)


def test_empty_batch_and_empty_range():
    wl = _wl(0, 64, 16, 2, 2, 4)
    shape = _shape(wl)
    pos = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    wo = torch.zeros((wl.W + 1,), dtype=torch.int32, device=DEV)
    two = torch.full((wl.W + 1,), -3, dtype=torch.int32, device=DEV)
    order = torch.empty((0,), dtype=torch.int32, device=DEV)
    moe.combine_order(pos, wo, shape, two, order)
    torch.cuda.synchronize()
    assert host(two).tolist() == [0] * (wl.W + 1)
    # w0 == w1: nothing written
    wl = CASES["one_wave"]
    x, idx, w = _inputs(wl)
    shape, out, eo, wd, y_ref = _run(wl, x, idx, w)
    two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
    y = torch.empty_like(y_ref)
    y.view(torch.uint8).fill_(0x33)
    moe.combine_waves(eo, wd, out["pos"], order, two, shape, 1, 1, y=y)
    torch.cuda.synchronize()
    assert bool((y.view(torch.uint8) == 0x33).all())


def test_full_size_dirichlet_waves():
    """T = 16384, H = 7168, E = 256, k = 8, W = 8: the order in full against the
    oracle, and the wave-by-wave combine equal to the one-pass combine on every
    token."""
    wl = synth.WORKLOADS["dirichlet_waves"]
    print(f"[combine waves] full size: T={wl.T} H={wl.H} E={wl.E} k={wl.k} W={wl.W}", flush=True)
    x, idx, w = _inputs(wl)
    shape, out, eo, wd, y_ref = _run(wl, x, idx, w)
    two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
    two_o, order_o = oracle.combine_order(idx, wl.E, wl.R, wl.W)
    np.testing.assert_array_equal(host(two), two_o)
    np.testing.assert_array_equal(host(order), order_o)
    y = torch.empty_like(y_ref)
    for w0 in range(wl.W):
        moe.combine_waves(eo, wd, out["pos"], order, two, shape, w0, w0 + 1, y=y)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))


def test_tables_out_of_range_are_clamped():
    """Offsets outside [0, T] and order entries that are not tokens: the wave
    combine clamps the range to [0, T] and skips the entries, writing only the
    listed tokens' rows (as moe_combine computes them)."""
    wl = CASES["k1"]
    x, idx, w = _inputs(wl)
    shape, out, eo, wd, y_ref = _run(wl, x, idx, w)
    T = wl.T
    order = torch.arange(T, dtype=torch.int32, device=DEV)
    order[::5] = -1
    order[1::7] = T + 3
    two = torch.tensor([-40] + [T // 2] * (wl.W - 1) + [T + 100], dtype=torch.int32, device=DEV)
    y = torch.empty_like(y_ref)
    y.view(torch.uint8).fill_(0x77)
    moe.combine_waves(eo, wd, out["pos"], order, two, shape, 0, wl.W, y=y)
    torch.cuda.synchronize()
    listed = torch.zeros(T, dtype=torch.bool, device=DEV)
    o = order.long()
    listed[o[(o >= 0) & (o < T)]] = True
    assert torch.equal(_bits(y[listed]), _bits(y_ref[listed]))
    assert bool((y.view(torch.uint8)[~listed] == 0x77).all())
    assert int(listed.sum()) < T

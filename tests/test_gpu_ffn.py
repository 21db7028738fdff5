"""Parity of the MFMA grouped SwiGLU expert FFN with the oracle, on the GPU.

The GPU accumulates in fp32 in MFMA order; the oracle in double. Both round the
intermediate h and the output to bf16. Bar: the element-wise rounding bound of
ffn_tolerance (fp32 accumulation of both GEMMs, the bf16 rounding flips of h
that the kernel's fp32 error allows, the output rounding), built from the
oracle's own sums; a wrong row, expert, weight or index shows up as errors of
the order of the outputs, far above it.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
from ffn_tolerance import check_rows, swiglu_rows_bound
import synth
from test_gpu_parity import dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ffn_setup(wl, std):
    logits, x = synth.logits(wl), synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=std)
    idx_o, w_o = oracle.route(logits, wl.k)
    ec, _ = oracle.counts(idx_o, wl.E, wl.R, wl.W)
    eo, _, _ = oracle.offsets(ec, wl.R, wl.W)
    nrows = int(ec.sum())
    pos, rt = oracle.positions(idx_o, wl.E, eo, nrows)
    return logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt


def _row_expert(ec, eo, rows):
    nonempty = np.nonzero(ec > 0)[0]
    starts = eo[nonempty]
    order = np.argsort(starts)
    return nonempty[order][np.searchsorted(starts[order], rows, side="right") - 1]


def _check_rows(got_bits, x_rows, row_expert, gu, dn, tight_atol=2e-3):
    """The GPU's expert rows against the oracle's within the rounding bound of
    ffn_tolerance (fp32 accumulation, bf16 rounding flips of h, output
    rounding), and all but a rare few within 2^-7 |out| + tight_atol."""
    o64, _, bound = swiglu_rows_bound(x_rows, row_expert, gu, dn)
    return check_rows(got_bits, o64, bound, tight_atol)


def _run_gpu(wl, x, gu, dn, idx_o, two_chains=True):
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    out = moe.dispatch(dev(x), dev(idx_o), wl.E, wl.R, wl.W)
    eo_gpu = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                               dev(gu), dev(dn), chains=moe.Chains() if two_chains else None)
    return shape, out, eo_gpu


@pytest.mark.parametrize("T,E,H,I,k,seed", [(300, 4, 256, 128, 2, 1), (77, 5, 128, 64, 3, 2),
                                            (1000, 16, 256, 192, 2, 3),
                                            (200, 3, 7168, 256, 2, 7),  # wide rows (H = 7168)
                                            (300, 1, 256, 128, 1, 8)])  # one expert
@pytest.mark.parametrize("two_chains", [True, False])
def test_swiglu_small_full(T, E, H, I, k, seed, two_chains):
    wl = synth.Workload("ffn", T=T, H=H, dtype="bf16", E=E, k=k, R=1, W=1, routing="zipf0.5",
                        expert="swiglu", I=I, seed=seed)
    print(f"[ffn] T={T} E={E} H={H} I={I} k={k} two_chains={two_chains}", flush=True)
    logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.1)
    shape, out, eo_gpu = _run_gpu(wl, x, gu, dn, idx_o, two_chains)
    torch.cuda.synchronize()
    nrows = int(ec.sum())
    rows = np.arange(nrows)
    _check_rows(host(eo_gpu), x[rt[rows]], _row_expert(ec, eo, rows), gu, dn)


@pytest.mark.parametrize("H,I", [(128, 64), (256, 128)])  # 128- and 256-row tile paths
def test_swiglu_empty_and_ragged_experts(H, I):
    # experts with 0, 1 and 257 rows (m-tile tails of both tile sizes), routed by hand
    E, k = 4, 1
    T = 259
    idx = np.zeros((T, k), np.int32)
    idx[:257, 0] = 2
    idx[257, 0] = 0
    idx[258, 0] = 3
    wl = synth.Workload("ffn", T=T, H=H, dtype="bf16", E=E, k=k, R=1, W=1, routing="iid",
                        expert="swiglu", I=I, seed=4)
    x = synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=0.1)
    ec, _ = oracle.counts(idx, E, 1, 1)
    eo, _, _ = oracle.offsets(ec, 1, 1)
    pos, rt = oracle.positions(idx, E, eo, T)
    shape, out, eo_gpu = _run_gpu(wl, x, gu, dn, idx)
    torch.cuda.synchronize()
    rows = np.arange(T)
    _check_rows(host(eo_gpu), x[rt], _row_expert(ec, eo, rows), gu, dn)


@pytest.mark.parametrize("two_chains", [True, False])
@pytest.mark.parametrize("H,I", [(128, 64), (256, 128)])  # 128- and 256-row tile paths
def test_swiglu_stores_stay_in_their_rows(H, I, two_chains):
    """The epilogue stores through buffer descriptors whose range check drops
    the rows past a tile's last one: with the last expert's tile mostly past
    the end of expert_out and of the h workspace, guard bytes right after both
    stay untouched, and every row is right."""
    E, k = 4, 1
    sizes = {0: 3, 1: 300, 3: 5}  # expert 2 has no rows; expert 3 (last) a 5-row tile
    T = sum(sizes.values())
    idx = np.concatenate([np.full(n, e, np.int32) for e, n in sizes.items()]).reshape(T, k)
    wl = synth.Workload("ffn", T=T, H=H, dtype="bf16", E=E, k=k, R=1, W=1, routing="iid",
                        expert="swiglu", I=I, seed=6)
    print(f"[ffn guard] H={H} I={I} two_chains={two_chains}", flush=True)
    x = synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=0.1)
    ec, _ = oracle.counts(idx, E, 1, 1)
    eo, _, _ = oracle.offsets(ec, 1, 1)
    pos, rt = oracle.positions(idx, E, eo, T)
    shape = moe.Shape(T, H, E, k, 1, 1, torch.bfloat16)
    out = moe.dispatch(dev(x), dev(idx), E, 1, 1)
    guard = 256  # rows past the end (a whole tile's worth)
    big_out = torch.empty((T * k + guard, H), dtype=torch.bfloat16, device=DEV)
    big_out.view(torch.uint8).fill_(0xA7)
    ws_bytes = moe.expert_swiglu_workspace_bytes(shape, I)
    big_ws = torch.empty((ws_bytes + guard * I * 2,), dtype=torch.uint8, device=DEV)
    big_ws.fill_(0x5C)
    eo_gpu = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                               dev(gu), dev(dn), expert_out=big_out[:T * k],
                               workspace=big_ws[:ws_bytes],
                               chains=moe.Chains() if two_chains else None)
    torch.cuda.synchronize()
    assert bool((big_out[T * k:].view(torch.uint8) == 0xA7).all())
    assert bool((big_ws[ws_bytes:] == 0x5C).all())
    rows = np.arange(T)
    _check_rows(host(eo_gpu), x[rt], _row_expert(ec, eo, rows), gu, dn)


def test_swiglu_validation():
    wl = synth.WORKLOADS["local_layer"]
    sh = moe.Shape(8, 4096, 16, 2, 1, 1, torch.bfloat16)
    assert moe.expert_swiglu_workspace_bytes(sh, 1408) == 16 * 1408 * 2
    assert moe.expert_swiglu_workspace_bytes(sh, 100) == 0
    t = torch.empty(16, dtype=torch.uint8, device=DEV)
    cs = sh.c()
    L = moe.lib()
    import ctypes
    P = ctypes.c_void_p(t.data_ptr())
    assert L.moe_expert_swiglu(ctypes.byref(cs), 100, P, P, P, P, P, P, P, 1 << 30, None, None, None, None) == -1
    sh32 = moe.Shape(8, 4096, 16, 2, 1, 1, torch.float32).c()
    assert L.moe_expert_swiglu(ctypes.byref(sh32), 1408, P, P, P, P, P, P, P, 1 << 30, None, None, None, None) == -4
    assert L.moe_expert_swiglu(ctypes.byref(cs), 1408, P, P, P, P, P, P, P, 10, None, None, None, None) == -3
    del wl


def test_local_layer_full_size_sampled():
    """The local-layer workload at full size (T=8192, E=16, H=4096, I=1408,
    weights N(0, 0.02^2)): FFN rows at both edges of every m-tile of every
    expert plus a random sample, and combined tokens end to end."""
    wl = synth.WORKLOADS["local_layer"]
    print(f"[ffn] local_layer full T={wl.T} H={wl.H} E={wl.E} I={wl.I}", flush=True)
    logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.02)
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    idx, w = moe.route(dev(logits), wl.k)
    out = moe.dispatch(dev(x), idx, wl.E, wl.R, wl.W)
    eo_gpu = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                               dev(gu), dev(dn), chains=moe.Chains())
    y = moe.combine(eo_gpu, w, out["pos"], shape)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), idx_o)
    np.testing.assert_array_equal(host(out["pos"]), pos)

    g = np.random.default_rng(7)
    # the first and last row of every 256-row m-tile of every expert (the
    # kernel's tile edges, partial last tiles included) and a random sample
    edges = []
    for e in np.nonzero(ec > 0)[0]:
        starts = np.arange(eo[e], eo[e] + ec[e], 256)
        edges += [starts, np.minimum(starts + 255, eo[e] + ec[e] - 1)]
    rows = np.unique(np.concatenate(edges + [g.integers(0, int(ec.sum()), 24)]))
    print(f"[ffn] local_layer full: {len(rows)} rows checked", flush=True)
    got = host(eo_gpu[torch.from_numpy(rows).to(DEV)])
    _check_rows(got, x[rt[rows]], _row_expert(ec, eo, rows), gu, dn, tight_atol=1e-3)

    # combined tokens: y_t = bf16(fp32 fma chain of w_ti * row_i) over the k
    # expert rows (stored in bf16). Against sum_i w_ti * out_f64 of the oracle,
    # each row carries its rounding bound B_i, the chain gamma_k and the fp32
    # weights (within 2^-23 relative of the oracle's), y its own rounding
    toks = np.unique(np.concatenate([[0, wl.T - 1], g.integers(0, wl.T, 6)]))
    y_ref = np.zeros((len(toks), wl.H))
    bound = np.zeros((len(toks), wl.H))
    for j, t in enumerate(toks):
        o64, _, b = swiglu_rows_bound(np.repeat(x[t:t + 1], wl.k, 0), idx_o[t], gu, dn)
        wt = w_o[t][:, None]
        y_ref[j] = (wt * o64).sum(0)
        e1 = (wt * b).sum(0) + (wl.k * 2.0**-24 + 2.0**-22) * (wt * (np.abs(o64) + b)).sum(0)
        bound[j] = e1 * (1 + 2.0**-8) + 2.0**-8 * np.abs(y_ref[j])
    yg = oracle.bf16_to_f64(host(y[torch.from_numpy(toks).to(DEV)]))
    err = np.abs(yg - y_ref)
    assert (err <= bound).all(), f"max combine err {err.max()}, err/bound {(err / bound).max()}"


def test_swiglu_chains_follow_caller_stream():
    """On a stream of the caller's own, with no synchronisation between calls:
    the side-stream chain must start after the dispatch queued before it and
    the combine queued after it must see both chains' rows."""
    wl = synth.Workload("ffn", T=2048, H=256, dtype="bf16", E=16, k=2, R=1, W=1,
                        routing="zipf0.5", expert="swiglu", I=192, seed=5)
    print(f"[ffn] caller stream: T={wl.T} E={wl.E} H={wl.H} I={wl.I}", flush=True)
    logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.1)
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    xd, gud, dnd, ld = dev(x), dev(gu), dev(dn), dev(logits)
    torch.cuda.synchronize()
    ref = None
    for attempt in range(2):
        s = torch.cuda.Stream()
        chains = moe.Chains()
        with torch.cuda.stream(s):
            idx, w = moe.route(ld, wl.k)
            out = moe.alloc_dispatch(shape, DEV)
            out["send_buf"].view(torch.uint8).fill_(0xA5)  # stale rows would show
            moe.dispatch_index(idx, shape, out)
            moe.dispatch_copy(xd, out["pos"], shape, out["send_buf"])
            eo_gpu = torch.empty_like(out["send_buf"])
            eo_gpu.view(torch.uint8).fill_(0x5A)
            moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                              gud, dnd, expert_out=eo_gpu, chains=chains)
            y = moe.combine(eo_gpu, w, out["pos"], shape)
            got = (eo_gpu.clone(), y.clone())
        s.synchronize()
        # the combine queued behind the FFN on the caller's stream must equal
        # one run after everything has finished
        y_after = moe.combine(got[0], w, out["pos"], shape)
        torch.cuda.synchronize()
        assert torch.equal(got[1].view(torch.uint8), y_after.view(torch.uint8))
        if ref is None:
            ref = got
            nrows = int(ec.sum())
            rows = np.arange(nrows)
            _check_rows(host(got[0]), x[rt[rows]], _row_expert(ec, eo, rows), gu, dn)
        else:  # a second stream, same results bit for bit
            assert torch.equal(got[0].view(torch.uint8), ref[0].view(torch.uint8))
            assert torch.equal(got[1].view(torch.uint8), ref[1].view(torch.uint8))


def test_swiglu_two_caller_streams_one_thread():
    """Two FFN calls in flight at once from one host thread, each on a stream of
    its own with its own side stream and events (the library keeps none): both
    equal the same calls run one after the other, bit for bit."""
    wls = [synth.Workload("ffn", T=T, H=256, dtype="bf16", E=E, k=2, R=1, W=1, routing="zipf0.5",
                          expert="swiglu", I=128, seed=seed)
           for T, E, seed in ((1536, 16, 21), (900, 8, 22))]
    print("[ffn] two caller streams: " + ", ".join(f"T={w.T} E={w.E}" for w in wls), flush=True)
    runs = []
    for wl in wls:
        logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.1)
        shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
        out = moe.dispatch(dev(x), dev(idx_o), wl.E, wl.R, wl.W)
        runs.append((wl, shape, out, dev(gu), dev(dn), x, gu, dn, ec, eo, rt))
    torch.cuda.synchronize()
    serial = []
    for wl, shape, out, gud, dnd, *_ in runs:
        serial.append(moe.expert_swiglu(out["send_buf"], out["expert_offsets"],
                                        out["expert_counts"], shape, gud, dnd,
                                        chains=moe.Chains()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    chains = [moe.Chains() for _ in runs]
    got = []
    for (wl, shape, out, gud, dnd, *_), s, ch in zip(runs, streams, chains):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            eo_gpu = torch.empty_like(out["send_buf"])
            eo_gpu.view(torch.uint8).fill_(0x5A)
            got.append(moe.expert_swiglu(out["send_buf"], out["expert_offsets"],
                                         out["expert_counts"], shape, gud, dnd, expert_out=eo_gpu,
                                         chains=ch))
    for s in streams:
        s.synchronize()
    for (wl, shape, out, gud, dnd, x, gu, dn, ec, eo, rt), a, b in zip(runs, got, serial):
        n = int(ec.sum())
        assert torch.equal(a[:n].view(torch.int16), b[:n].view(torch.int16))
        rows = np.arange(n)
        _check_rows(host(a)[:n], x[rt[rows]], _row_expert(ec, eo, rows), gu, dn)

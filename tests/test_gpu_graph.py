"""The library's calls captured in one HIP graph (torch.cuda.graph on a side
stream) and replayed: every replay must reproduce the eager results bit for
bit. Replays are separated by eager work on other buffers and by
synchronisations, and every output is overwritten with garbage before each
replay, so a replay that skipped or repeated a node would show. No kernel of
the library clears memory with a runtime memset, which is what graph replays
can get wrong; this checks the whole step as captured."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import synth
from test_gpu_parity import DEV, PARITY, dev, shape_of

pytestmark = pytest.mark.gpu


def _replays_match(step, outputs, eager_noise):
    """Eager reference, then capture, then three replays checked one by one."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}, output {i}"


def test_graph_replay_default_step():
    wl = PARITY["zipf"]
    print(f"[graph] zipf step: T={wl.T} H={wl.H} E={wl.E} k={wl.k}", flush=True)
    shape = shape_of(wl)
    logits, x = dev(synth.logits(wl)), dev(synth.hidden(wl))
    out = moe.alloc_dispatch(shape, DEV)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    raw = torch.empty((moe.STATS_BYTES,), dtype=torch.uint8, device=DEV)
    eo = torch.empty_like(out["send_buf"])
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    # eager work between replays: the same path on a second set of buffers
    out2 = moe.alloc_dispatch(shape, DEV)
    idx2, w2 = torch.empty_like(idx), torch.empty_like(w)

    def step():
        moe.route_index(logits, shape, out, idx, w, stats_out=raw)
        moe.dispatch_copy(x, out["pos"], shape, out["send_buf"])
        moe.expert_scale(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                         expert_out=eo)
        moe.combine(eo, w, out["pos"], shape, y=y)

    def noise():
        moe.route_index(logits, shape, out2, idx2, w2)
        moe.dispatch_copy(x, out2["pos"], shape, out2["send_buf"])

    n = wl.T * wl.k
    outputs = [idx, w, raw, out["expert_counts"], out["expert_offsets"], out["rank_counts"],
               out["rank_offsets"], out["wave_offsets"], out["pos"], out["row_token"][:n],
               out["send_buf"], eo, y]
    _replays_match(step, outputs, noise)


def test_graph_replay_decode_step():
    """The decode step as the benchmark's --fused path runs it: routing, the
    one-launch dispatch with its statistics block, experts, combine; and the
    wave-pipelined identity-scaled experts on two streams with the per-wave
    combine on a third (dirichlet_waves layout, W = 8) in the same graph."""
    wl = synth.WORKLOADS["decode_hot"]
    print(f"[graph] decode step: T={wl.T} H={wl.H} E={wl.E} k={wl.k}", flush=True)
    shape = shape_of(wl)
    logits, x = dev(synth.logits(wl)), dev(synth.hidden(wl))
    out = moe.alloc_dispatch(shape, DEV)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    raw = torch.empty((moe.STATS_BYTES,), dtype=torch.uint8, device=DEV)
    eo = torch.empty_like(out["send_buf"])
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    wv = synth.WORKLOADS["dirichlet_waves"].with_(T=256, H=512)
    shape_w = shape_of(wv)
    logits_w, x_w = dev(synth.logits(wv)), dev(synth.hidden(wv))
    out_w = moe.alloc_dispatch(shape_w, DEV)
    idx_w = torch.empty((wv.T, wv.k), dtype=torch.int32, device=DEV)
    w_w = torch.empty((wv.T, wv.k), dtype=torch.float32, device=DEV)
    eo_w = torch.empty_like(out_w["send_buf"])
    y_w = torch.empty((wv.T, wv.H), dtype=torch.bfloat16, device=DEV)
    two_w = torch.empty((wv.W + 1,), dtype=torch.int32, device=DEV)
    order_w = torch.empty((wv.T,), dtype=torch.int32, device=DEV)
    copy, cstream = torch.cuda.Stream(), torch.cuda.Stream()
    chains = moe.Chains(n_events=moe.scale_waves_events(wv.W), side=False)
    out2 = moe.alloc_dispatch(shape, DEV)
    idx2, w2 = torch.empty_like(idx), torch.empty_like(w)

    def step():
        moe.route_dispatch(logits, x, shape, out, idx, w, stats=raw)
        moe.expert_scale(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                         expert_out=eo)
        moe.combine(eo, w, out["pos"], shape, y=y)
        moe.route_index(logits_w, shape_w, out_w, idx_w, w_w)
        moe.combine_order(out_w["pos"], out_w["wave_offsets"], shape_w, two_w, order_w)
        moe.scale_waves(x_w, out_w, shape_w, expert_out=eo_w, copy_stream=copy, chains=chains,
                        combine=dict(topk_w=w_w, pos=out_w["pos"], token_order=order_w,
                                     token_wave_offsets=two_w, y=y_w, stream=cstream))

    def noise():
        moe.route_dispatch(logits, x, shape, out2, idx2, w2)

    n, nw = wl.T * wl.k, wv.T * wv.k
    outputs = [idx, w, raw, out["expert_counts"], out["expert_offsets"], out["rank_counts"],
               out["rank_offsets"], out["wave_offsets"], out["pos"], out["row_token"][:n],
               out["send_buf"], eo, y, out_w["send_buf"][:nw], eo_w[:nw], y_w, two_w, order_w]
    _replays_match(step, outputs, noise)


def test_graph_replay_capacity_and_direct_exchange():
    wl = PARITY["zipf"]
    print(f"[graph] capacity + direct exchange: T={wl.T} H={wl.H} E={wl.E}", flush=True)
    shape = shape_of(wl)
    logits, x = dev(synth.logits(wl)), dev(synth.hidden(wl))
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    cap = moe.expert_capacity(wl.k, 1.0, wl.T, wl.E)
    cb = moe.alloc_dispatch_capacity(shape, cap, DEV)
    vb = moe.alloc_vsrc(shape, DEV)
    shape1 = shape_of(wl.with_(W=1))
    veo = torch.empty_like(vb["send_buf"])
    back = torch.empty_like(vb["send_buf"])
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)

    def step():
        moe.route(logits, wl.k, topk_idx=idx, topk_w=w)
        moe.dispatch_capacity(x, idx, wl.E, wl.R, wl.W, cap, out=cb)
        moe.vsrc_dispatch(x, idx, shape, vb)
        moe.vsrc_exchange_direct(vb["send_buf"], vb["grouped"], shape, vb, 0)
        moe.expert_scale_rows(vb["grouped"], vb["expert_offsets"], vb["expert_counts"], shape1,
                              expert_out=veo)
        moe.vsrc_exchange_direct(veo, back, shape, vb, 1)
        moe.combine_rows(back, w, vb["pos"], shape, y=y)

    def noise():
        moe.route(logits, wl.k)

    n = int(np.prod(idx.shape))
    outputs = [idx, w, cb["kept_counts"], cb["pos"], cb["row_token"], cb["send_buf"],
               vb["src_counts"], vb["src_offsets"], vb["send_counts"], vb["recv_offsets"],
               vb["expert_offsets"], vb["pos"], vb["send_buf"][:n], vb["grouped"][:n], y]
    _replays_match(step, outputs, noise)


def test_graph_replay_exchange_and_regroup():
    """The emulated exchange the long way: all-to-all, regroup, experts,
    ungroup, reverse all-to-all, combine (segment copies storing through the
    caches)."""
    wl = PARITY["zipf"]
    print(f"[graph] exchange + regroup: T={wl.T} H={wl.H} E={wl.E} R={wl.R}", flush=True)
    shape = shape_of(wl)
    logits, x = dev(synth.logits(wl)), dev(synth.hidden(wl))
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    vb = moe.alloc_vsrc(shape, DEV)
    shape1 = shape_of(wl.with_(W=1))
    veo = torch.empty_like(vb["send_buf"])
    ung = torch.empty_like(vb["send_buf"])
    back = torch.empty_like(vb["send_buf"])
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)

    def step():
        moe.route(logits, wl.k, topk_idx=idx, topk_w=w)
        moe.vsrc_dispatch(x, idx, shape, vb)
        moe.vsrc_exchange(vb["send_buf"], vb["recv_buf"], shape, vb, 0)
        moe.vsrc_regroup(vb["recv_buf"], vb["grouped"], shape, vb, 0)
        moe.expert_scale_rows(vb["grouped"], vb["expert_offsets"], vb["expert_counts"], shape1,
                              expert_out=veo)
        moe.vsrc_regroup(veo, ung, shape, vb, 1)
        moe.vsrc_exchange(ung, back, shape, vb, 1)
        moe.combine_rows(back, w, vb["pos"], shape, y=y)

    def noise():
        moe.route(logits, wl.k)

    n = int(np.prod(idx.shape))
    outputs = [idx, w, vb["recv_counts"], vb["recv_offsets"], vb["send_buf"][:n],
               vb["recv_buf"][:n], vb["grouped"][:n], veo[:n], back[:n], y]
    _replays_match(step, outputs, noise)


def test_graph_replay_swiglu_chains():
    """The SwiGLU FFN forks its odd-id experts onto the caller's side stream and
    joins them back: captured, the fork and join become graph edges."""
    wl = synth.Workload("ffn", T=1000, H=256, dtype="bf16", E=16, k=2, R=1, W=1,
                        routing="zipf0.5", expert="swiglu", I=192, seed=3)
    print(f"[graph] swiglu: T={wl.T} H={wl.H} E={wl.E} I={wl.I} k={wl.k}", flush=True)
    shape = shape_of(wl)
    x = dev(synth.hidden(wl))
    gu, dn = (dev(a) for a in synth.swiglu_weights(wl, std=0.1))
    idx, _ = moe.route(dev(synth.logits(wl)), wl.k)
    out = moe.dispatch(x, idx, wl.E, wl.R, wl.W)
    eo = torch.empty_like(out["send_buf"])
    ws = torch.empty((moe.expert_swiglu_workspace_bytes(shape, wl.I),), dtype=torch.uint8,
                     device=DEV)
    eo2, ws2 = torch.empty_like(eo), torch.empty_like(ws)
    chains, chains2 = moe.Chains(), moe.Chains()

    def step():
        moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                          gu, dn, expert_out=eo, workspace=ws, chains=chains)

    def noise():  # the same FFN eagerly, through another side stream
        moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                          gu, dn, expert_out=eo2, workspace=ws2, chains=chains2)

    _replays_match(step, [eo], noise)
    assert torch.equal(eo2.view(torch.uint8), eo.view(torch.uint8))


def test_graph_swiglu_first_call_captured():
    """The very first call with a fresh side stream and events is made inside
    a capture (nothing in the library is set up on first use): the replays
    equal an eager run made afterwards, bit for bit."""
    wl = synth.Workload("ffn", T=700, H=256, dtype="bf16", E=8, k=2, R=1, W=1,
                        routing="zipf0.5", expert="swiglu", I=128, seed=9)
    print(f"[graph] swiglu first call: T={wl.T} H={wl.H} E={wl.E} I={wl.I}", flush=True)
    shape = shape_of(wl)
    x = dev(synth.hidden(wl))
    gu, dn = (dev(a) for a in synth.swiglu_weights(wl, std=0.1))
    idx, _ = moe.route(dev(synth.logits(wl)), wl.k)
    out = moe.dispatch(x, idx, wl.E, wl.R, wl.W)
    eo = torch.empty_like(out["send_buf"])
    ws = torch.empty((moe.expert_swiglu_workspace_bytes(shape, wl.I),), dtype=torch.uint8,
                     device=DEV)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        chains = moe.Chains()  # created outside the capture, used first inside it
    cap.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"],
                              shape, gu, dn, expert_out=eo, workspace=ws, chains=chains)
    torch.cuda.synchronize()
    ref = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                            gu, dn, chains=moe.Chains())
    torch.cuda.synchronize()
    n = int(out["expert_counts"].sum().item())
    for rep in range(3):
        eo.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(eo[:n].view(torch.uint8), ref[:n].view(torch.uint8)), rep

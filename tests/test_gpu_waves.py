"""Wave-pipelined local layer (irregular AllToAll page, wave-scheduled
pipelining) through the C ABI: per wave a gather dispatch of the wave's rows on
a copy stream and the SwiGLU FFN of the wave's experts on the compute stream.

Bars: the gathered send rows bit-exact against the oracle's dispatch; the
expert rows bit-identical to the unpipelined moe_expert_swiglu on the same send
buffer (same per-element MFMA arithmetic) and within the FFN tolerance of the
oracle's fp64 SwiGLU (its rounding bound); the combined tokens bit-identical to
the unpipelined path, also when each wave's completed tokens are combined in
the pipeline."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_ffn import _check_rows, _row_expert
from test_gpu_parity import DEV, dev, host

pytestmark = pytest.mark.gpu


def _setup(wl, std=0.1):
    logits, x = synth.logits(wl), synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=std)
    idx, w = oracle.route(logits, wl.k)
    return x, gu, dn, idx, w


def _plain(wl, x, gu, dn, idx, w):
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    out = moe.dispatch(dev(x), dev(idx), wl.E, wl.R, wl.W)
    eo = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                           dev(gu), dev(dn), chains=moe.Chains())
    y = moe.combine(eo, dev(w.astype(np.float32)), out["pos"], shape)
    return shape, out, eo, y


def _waves(wl, x, gu, dn, idx, w, two_streams, side=True, in_pipe=None):
    """two_streams: gathers on a copy stream; side: the caller's side stream
    for the second chain of a wave's experts (with neither, no events at all);
    in_pipe: each wave's completed tokens combined in the pipeline instead of
    one combine afterwards, on the copy stream ("copy") or on a stream of their
    own ("own")."""
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    out = moe.alloc_dispatch(shape, DEV)
    out["send_buf"].fill_(0)
    moe.dispatch_index(dev(idx), shape, out)
    copy = torch.cuda.Stream() if two_streams else None
    chains = (moe.Chains(n_events=moe.swiglu_waves_events(wl.W), side=side)
              if two_streams or side or in_pipe == "own" else None)
    xd, wd = dev(x), dev(w.astype(np.float32))
    if in_pipe:
        two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
        y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        comb = dict(topk_w=wd, pos=out["pos"], token_order=order, token_wave_offsets=two, y=y)
        if in_pipe == "own":
            comb["stream"] = torch.cuda.Stream()
        eo, y = moe.swiglu_waves(xd, out, shape, dev(gu), dev(dn), copy_stream=copy,
                                 chains=chains, combine=comb)
    else:
        eo = moe.swiglu_waves(xd, out, shape, dev(gu), dev(dn), copy_stream=copy, chains=chains)
        y = moe.combine(eo, wd, out["pos"], shape)
    torch.cuda.synchronize()
    return out, eo, y


# two chains of experts a wave: R1_W1, R1_W2 (one rank), R4_W1 (one wave); the
# others one chain (fewer than eight experts a wave, or a split that is not a
# stride-2 run of expert ids)
CASES = [("R1_W1", 1, 1), ("R1_W2", 1, 2), ("R1_W4", 1, 4), ("R1_W16", 1, 16), ("R2_W2", 2, 2),
         ("R4_W4", 4, 4), ("R4_W1", 4, 1)]


@pytest.mark.parametrize("name,R,W", CASES)
@pytest.mark.parametrize("two_streams,side,in_pipe", [
    (True, True, None), (False, True, None), (False, False, None), (True, True, "copy"),
    (False, False, "copy"), (True, True, "own"), (False, False, "own")])
def test_wave_pipeline_matches_plain_and_oracle(name, R, W, two_streams, side, in_pipe):
    wl = synth.WORKLOADS["local_layer"].with_(T=1024, H=256, I=128, R=R, W=W, seed=11)
    print(f"[waves] {name} two_streams={two_streams} side={side} in_pipe={in_pipe}: T={wl.T} "
          f"H={wl.H} E={wl.E} I={wl.I}", flush=True)
    x, gu, dn, idx, w = _setup(wl)
    shape, plain, eo_p, y_p = _plain(wl, x, gu, dn, idx, w)
    out, eo, y = _waves(wl, x, gu, dn, idx, w, two_streams, side, in_pipe)
    ref = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
    n = ref["nrows"]
    np.testing.assert_array_equal(host(out["send_buf"])[:n], ref["send_buf"])
    assert torch.equal(eo[:n], eo_p[:n])
    assert torch.equal(y, y_p)
    rows = np.arange(n)
    _check_rows(host(eo)[:n], x[ref["row_token"]], _row_expert(
        ref["expert_counts"], ref["expert_offsets"], rows), gu, dn)


@pytest.mark.parametrize("in_pipe", [False, True])
def test_wave_pipeline_full_size_repeat(in_pipe):
    """The local layer at full size, W = 4 on two streams (with in_pipe each
    wave's completed tokens combined on a third), twice in a row into the same
    buffers: identical to the unpipelined path both times."""
    wl = synth.WORKLOADS["local_layer"].with_(W=4)
    print(f"[waves full] T={wl.T} H={wl.H} E={wl.E} I={wl.I} W={wl.W} in_pipe={in_pipe}",
          flush=True)
    x, gu, dn, idx, w = _setup(wl, std=0.02)
    shape, plain, eo_p, y_p = _plain(wl, x, gu, dn, idx, w)
    out = moe.alloc_dispatch(shape, DEV)
    moe.dispatch_index(dev(idx), shape, out)
    side = torch.cuda.Stream()
    chains = moe.Chains(n_events=moe.swiglu_waves_events(wl.W))
    xd, gud, dnd = dev(x), dev(gu), dev(dn)
    eo = torch.empty_like(out["send_buf"])
    ws = torch.empty((moe.expert_swiglu_workspace_bytes(shape, wl.I),), dtype=torch.uint8,
                     device=DEV)
    n = int(host(out["expert_counts"]).sum())
    wd = dev(w.astype(np.float32))
    two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    comb = dict(topk_w=wd, pos=out["pos"], token_order=order, token_wave_offsets=two, y=y,
                stream=torch.cuda.Stream())
    for rep in range(2):
        eo.fill_(0)
        y.fill_(float("nan"))
        if in_pipe:
            moe.swiglu_waves(xd, out, shape, gud, dnd, expert_out=eo, workspace=ws,
                             copy_stream=side, chains=chains, combine=comb)
        else:
            moe.swiglu_waves(xd, out, shape, gud, dnd, expert_out=eo, workspace=ws,
                             copy_stream=side, chains=chains)
            moe.combine(eo, wd, out["pos"], shape, y=y)
        torch.cuda.synchronize()
        assert torch.equal(out["send_buf"][:n], plain["send_buf"][:n]), rep
        assert torch.equal(eo[:n], eo_p[:n]), rep
        assert torch.equal(y, y_p), rep


# ------------------------------------------- identity-scaled experts in waves

SCALE_CASES = [("dirichlet_shape_W8", 32, 8, 1024, 256), ("dirichlet_shape_W1", 32, 1, 1024, 256),
               ("R4_W2_f32", 4, 2, 700, 64), ("R1_W4_ragged", 1, 4, 333, 128)]


@pytest.mark.parametrize("name,R,W,T,H", SCALE_CASES)
@pytest.mark.parametrize("two_streams,in_pipe", [(True, None), (False, None), (True, "copy"),
                                                 (False, "copy"), (True, "own"), (False, "own")])
def test_scale_waves_match_plain(name, R, W, T, H, two_streams, in_pipe):
    """moe_scale_waves (per wave: gather dispatch on a copy stream, the wave's
    identity-scaled experts on the compute stream, with in_pipe the combine of
    the wave's completed tokens) against moe_dispatch_copy + moe_expert_scale
    + moe_combine and the oracle: send rows, expert rows and the combined
    tokens, bit for bit."""
    base = synth.WORKLOADS["dirichlet_waves"] if R == 32 else synth.WORKLOADS["zipf"]
    dt = "f32" if name.endswith("f32") else "bf16"
    E = 256 if R == 32 else 64
    wl = base.with_(T=T, H=H, E=E, R=R, W=W, dtype=dt, seed=7)
    print(f"[scale waves] {name} two_streams={two_streams} in_pipe={in_pipe}: T={T} H={H} E={E} "
          f"k={wl.k} R={R} W={W} {dt}", flush=True)
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx, w = oracle.route(logits, wl.k)
    ref = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
    out_o = oracle.expert_scale(ref["send_buf"], ref["expert_offsets"], ref["expert_counts"])
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    shape = moe.Shape(T, H, E, wl.k, R, W, tdt)
    xd, idd, wd = dev(x), dev(idx), dev(w.astype(np.float32))
    plain = moe.dispatch(xd, idd, E, R, W)
    eo_p = moe.expert_scale(plain["send_buf"], plain["expert_offsets"], plain["expert_counts"],
                            shape)
    y_p = moe.combine(eo_p, wd, plain["pos"], shape)
    out = moe.alloc_dispatch(shape, DEV)
    moe.dispatch_index(idd, shape, out)
    out["send_buf"].view(torch.uint8).fill_(0xA5)
    eo = torch.empty_like(out["send_buf"])
    eo.view(torch.uint8).fill_(0x5A)
    copy = torch.cuda.Stream() if two_streams else None
    chains = (moe.Chains(n_events=moe.scale_waves_events(W), side=False)
              if two_streams or in_pipe == "own" else None)
    if in_pipe:
        two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
        y = torch.empty((T, H), dtype=tdt, device=DEV)
        y.view(torch.uint8).fill_(0xA5)
        comb = dict(topk_w=wd, pos=out["pos"], token_order=order, token_wave_offsets=two, y=y)
        if in_pipe == "own":
            comb["stream"] = torch.cuda.Stream()
        moe.scale_waves(xd, out, shape, expert_out=eo, copy_stream=copy, chains=chains,
                        combine=comb)
    else:
        moe.scale_waves(xd, out, shape, expert_out=eo, copy_stream=copy, chains=chains)
        y = moe.combine(eo, wd, out["pos"], shape)
    torch.cuda.synchronize()
    n = ref["nrows"]
    np.testing.assert_array_equal(host(out["send_buf"])[:n], ref["send_buf"])
    np.testing.assert_array_equal(host(eo)[:n], out_o)
    bits = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(eo[:n].view(bits), eo_p[:n].view(bits))
    assert torch.equal(y.view(bits), y_p.view(bits))


def test_scale_waves_full_size_dirichlet_waves():
    """dirichlet_waves at full size (T=16384, H=7168, E=256, k=8, R=32, W=8): the
    wave pipeline on two streams with each wave's completed tokens combined on
    a third, bit for bit against moe_dispatch_copy + moe_expert_scale +
    moe_combine on every send row, expert row and token."""
    wl = synth.WORKLOADS["dirichlet_waves"]
    print(f"[scale waves full] T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} W={wl.W}",
          flush=True)
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    logits, xd = dev(synth.logits(wl)), dev(synth.hidden(wl))
    idx, wd = moe.route(logits, wl.k)
    plain = moe.dispatch(xd, idx, wl.E, wl.R, wl.W)
    eo_p = moe.expert_scale(plain["send_buf"], plain["expert_offsets"], plain["expert_counts"],
                            shape)
    y_p = moe.combine(eo_p, wd, plain["pos"], shape)
    out = moe.alloc_dispatch(shape, DEV)
    moe.dispatch_index(idx, shape, out)
    two, order = moe.combine_order(out["pos"], out["wave_offsets"], shape)
    eo = torch.empty_like(out["send_buf"])
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    chains = moe.Chains(n_events=moe.scale_waves_events(wl.W), side=False)
    moe.scale_waves(xd, out, shape, expert_out=eo, copy_stream=torch.cuda.Stream(), chains=chains,
                    combine=dict(topk_w=wd, pos=out["pos"], token_order=order,
                                 token_wave_offsets=two, y=y, stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    n = wl.T * wl.k
    assert torch.equal(out["send_buf"][:n].view(torch.int16), plain["send_buf"][:n].view(torch.int16))
    assert torch.equal(eo[:n].view(torch.int16), eo_p[:n].view(torch.int16))
    assert torch.equal(y.view(torch.int16), y_p.view(torch.int16))

"""The allocation-free dispatch entry point (moe_dispatch_noalloc) through the C
ABI against moe_dispatch, the entry point it varies: every output bit for bit,
on calls in a row into the library's one static scratch array, each using less
of it than the one before (so stale histogram rows of a larger call are
present): first E = 1024 with 65536 picks, whose histogram fills the array
exactly, then the largest configuration (dirichlet_waves, full size), then
smaller ones down to the tiny workload."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "wave_offsets", "pos",
        "row_token")


def _inputs(wl, T):
    idx, _ = oracle.route(synth.logits(wl, T), wl.k)
    x = synth.hidden(wl, T)
    xt = torch.from_numpy(np.ascontiguousarray(x).view(np.int16 if x.dtype == np.uint16 else
                                                       np.float32)).to(DEV)
    if x.dtype == np.uint16:
        xt = xt.view(torch.bfloat16)
    return xt, torch.from_numpy(idx).to(DEV)


def _fill(out):
    for v in out.values():
        v.view(torch.uint8).fill_(0xA5)


def test_noalloc_matches_dispatch_in_a_row():
    dirichlet = synth.WORKLOADS["dirichlet_waves"]
    wide = synth.Workload("wide", T=8192, H=128, dtype="f32", E=1024, k=8, R=8, W=2,
                          routing="iid", seed=5)
    cases = [(wide, wide.T), (dirichlet, dirichlet.T), (synth.WORKLOADS["zipf"], 4096),
             (synth.WORKLOADS["zipf"], 777), (synth.WORKLOADS["tiny"], 256)]
    assert moe.noalloc_scratch_bytes() == 256 << 10
    used = None
    for wl, T in cases:
        # histogram bytes this call uses: chunks x E int32 (1024-pick chunks, at
        # most 65536 / pow2(E) of them)
        picks = T * wl.k
        pow2 = 1 << (wl.E - 1).bit_length()
        max_chunks = min(512, 65536 // pow2)
        chunk = max(1024, -(-(-(-picks // max_chunks)) // 1024) * 1024)
        hist = -(-picks // chunk) * wl.E * 4
        assert hist <= 256 << 10 and (used is None or hist < used)
        used = hist
        shape = moe.Shape(T, wl.H, wl.E, wl.k, wl.R, wl.W,
                          torch.float32 if wl.dtype == "f32" else torch.bfloat16)
        print(f"[noalloc] {wl.name} T={T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} W={wl.W}; "
              f"histogram {hist} B", flush=True)
        x, idx = _inputs(wl, T)
        ref = moe.alloc_dispatch(shape, DEV)
        moe.dispatch(x, idx, wl.E, wl.R, wl.W, out=ref)
        got = moe.alloc_dispatch(shape, DEV)
        del got["workspace"]
        _fill(got)
        moe.dispatch_noalloc(x, idx, shape, got)
        torch.cuda.synchronize()
        rows = int(ref["expert_counts"].sum().item())
        for key in KEYS:
            a, b = got[key], ref[key]
            if key == "row_token":
                a, b = a[:rows], b[:rows]
            assert torch.equal(a, b), f"{wl.name} T={T}: {key} differs from moe_dispatch"
        assert torch.equal(got["send_buf"][:rows].view(torch.int16 if x.dtype == torch.bfloat16
                                                        else torch.int32),
                           ref["send_buf"][:rows].view(torch.int16 if x.dtype == torch.bfloat16
                                                       else torch.int32)), f"{wl.name} T={T}"


def test_noalloc_validation_before_any_launch():
    L = moe.lib()
    import ctypes
    wl = synth.WORKLOADS["zipf"]
    sh = moe.Shape(64, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16).c()
    t = torch.empty(16, dtype=torch.int32, device=DEV)
    P = ctypes.c_void_p(t.data_ptr())
    assert L.moe_dispatch_noalloc(ctypes.byref(sh), P, P, P, None, P, P, P, P, P, P, None) == -1
    bad = moe.Shape(64, 100, wl.E, wl.k, wl.R, wl.W, torch.bfloat16).c()  # 200-byte rows
    assert L.moe_dispatch_noalloc(ctypes.byref(bad), P, P, P, P, P, P, P, P, P, P, None) == -2

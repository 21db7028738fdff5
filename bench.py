#!/usr/bin/env python3
"""Benchmark of the one-GPU MoE routing path on an MI355X.

One step = the whole path on one batch of synthetic input, inputs already in
HBM: route (top-k gating) -> dispatch index (counting pass, offsets,
positions) -> dispatch copy (permute into the send buffer) -> experts
(identity-scaled, or the SwiGLU FFN on MFMA for the local-layer workload) ->
combine -> skew statistics of S (moe_route, moe_dispatch, the expert call,
moe_combine, moe_stats: 7 kernels a step, or 5 when all T*k picks fit one
1024-pick batch, the decode regime, where moe_dispatch is one launch). With
--fused, routing, index, statistics and the dispatch copy go through
moe_route_dispatch instead (2 launches in the decode regime, else the routing
kernel with the counting pass, the placing kernel with the statistics block
and the copy; the counting pass then sits outside the dispatch+combine
region). Every step runs in the library's HIP kernels on torch's current
stream; torch only provides memory and the stream.

Prints ONE JSON line. `value` is the metric: dispatch+combine tokens/s, i.e. T
over the median (over steps) of the summed execution times of the dispatch
kernels (count, place, copy) and the combine kernel. Those come from an
instrumented K-step loop: the library's timing hook launches every kernel with
start/stop events (extended launches on the launch stream), so a stage's time
is its kernels' execution time. `ms_per_step` is the wall clock of K
uninstrumented whole steps (bracketed by synchronisations); a third loop runs
only the dispatch and combine calls K times for their wall clock. The dominant
dispatch/combine kernel's algorithmic bytes over its average duration is
`roofline` (the expert stage, outside the metric, has its own record). A
further loop repeats the instrumented steps after evicting the 256 MB Infinity
Cache (a 512 MiB scratch write) for cold-cache stage times.

--vsrc runs the exchange of R ranks emulated on the one device instead: every
source shard's dispatch and the count exchange, the block-transpose all-to-all,
the receive-side regroup, the experts on the regrouped rows, then ungroup,
reverse all-to-all and combine at the sources (15 kernels a step).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/sec and achieved HBM GB/s (% of peak) on 1 MI355X"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
STAGES = ("route", "dispatch", "dispatch_index", "dispatch_copy", "exchange", "regroup", "expert",
          "combine", "stats")
# The metric's region: counts, offsets, positions, the permute copy (and, for
# the emulated exchange, the exchange and regroup copies), and the combine.
# "dispatch" is the one-launch form of index + copy (T*k <= 1024).
DC_STAGES = ("dispatch", "dispatch_index", "dispatch_copy", "exchange", "regroup", "combine")


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded (same soname)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(out), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return out.value


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dirichlet_waves")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-evicted loop")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--graph", action="store_true",
                    help="also time K steps replayed from one captured HIP graph")
    ap.add_argument("--fused", action="store_true",
                    help="route, index, statistics and the dispatch copy through "
                         "moe_route_dispatch (two launches when T*k <= 1024, else three; the "
                         "counting pass then runs inside the routing kernel)")
    ap.add_argument("--wave-sweep", action="store_true",
                    help="wave-pipelined dispatch + experts for every W dividing L, two streams "
                         "vs one, with and without the per-wave combine; T(W) and the fitted "
                         "wave model")
    ap.add_argument("--waves", type=int, default=None,
                    help="with --wave-sweep: only this W (for a profiled run)")
    ap.add_argument("--vsrc", action="store_true",
                    help="the expert-parallel exchange of R virtual source ranks on one device")
    ap.add_argument("--direct", action="store_true",
                    help="with --vsrc: the exchange straight into the grouped layout (one copy "
                         "each way) instead of all-to-all + regroup")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="capacity-factor dispatch (buckets of ceil(k*f*T/E) rows, overflow "
                         "dropped, zero padding) instead of count-sized buckets")
    return ap.parse_args()


def algorithmic_bytes(wl) -> dict:
    """Minimum HBM bytes each stage must move per launch (b = element bytes)."""
    T, H, E, k, b = wl.T, wl.H, wl.E, wl.k, wl.elem_bytes
    out = {
        "route": T * E * 4 + T * k * 8,                          # logits in; idx + w out
        "dispatch_index": 12 * T * k + 4 * E,                    # idx in; pos, row_token, S out
        # (fused path: the counting pass moves no HBM bytes beyond route's)
        "stats": 4 * E,                                          # S in
        "dispatch_copy": T * H * b + T * k * H * b + 4 * T * k,  # x once, k copies, pos
        "expert": 2 * T * k * H * b,                             # rows in, rows out
        "combine": T * k * H * b + 8 * T * k + T * H * b,        # k rows, w + pos in; y out
    }
    out["dispatch"] = out["dispatch_index"] + out["dispatch_copy"]
    if wl.expert == "swiglu":  # + the expert weights, read once
        out["expert"] += 3 * wl.E * wl.H * wl.I * 2
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def source_code_hash(text: str) -> str:
    """First 16 hex digits of the SHA-256 of C/C++ source text with its comments
    and whitespace taken out, so that edits to comments alone keep a record."""
    import hashlib
    import re
    code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", text, flags=re.S)
    return hashlib.sha256(" ".join(code.split()).encode()).hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by the counters' reading of a plain 1 GiB copy),
    or None when there is no record or the code of the kernel's sources (their
    text without comments) changed since."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    fields = lambda ln: dict(kv.split("=", 1) for kv in ln.split()[1:])  # noqa: E731
    scale = next((fields(ln) for ln in lines if ln.startswith("scale ")), None)
    for ln in lines:
        if not ln.startswith("traffic "):
            continue
        f = fields(ln)
        if f.get("workload") != workload or f.get("kernel") != kernel or scale is None:
            continue
        text = ""
        for src in f["sources"].split(","):
            with open(os.path.join(ROOT, "combine_moe_route_03_amd", "csrc", src)) as fh:
                text += fh.read() + "\n"
        if source_code_hash(text) != f["code_sha256"]:
            return None
        kib = float(f["fetch_kib"]) * float(scale["fetch"]) + float(f["write_kib"]) * float(scale["write"])
        return int(round(kib * 1024))
    return None


def capacity_bytes(wl, cap: int, kept: int) -> dict:
    """The byte model with capacity-factor buckets: the copy writes every bucket
    row (kept rows and zero padding); experts and combine touch the kept rows."""
    T, H, E, k, b = wl.T, wl.H, wl.E, wl.k, wl.elem_bytes
    out = algorithmic_bytes(wl)
    out["dispatch_copy"] = T * H * b + E * cap * H * b + 4 * T * k
    out["expert"] = 2 * kept * H * b
    out["combine"] = kept * H * b + 8 * T * k + T * H * b
    return out


def vsrc_bytes(wl, nrows: int) -> dict:
    """The byte model of the emulated exchange: each exchange and regroup
    launch reads and writes every sent row once (two launches each a step)."""
    H, b = wl.H, wl.elem_bytes
    out = algorithmic_bytes(wl)
    out["exchange"] = 2 * 2 * nrows * H * b
    out["regroup"] = 2 * 2 * nrows * H * b
    return out


def ffn_flops(wl) -> int:
    return 6 * wl.T * wl.k * wl.H * wl.I  # gate/up (2*2I*H) + down (2*H*I) per row


def host_description() -> dict:
    """CPU model and the core counts of the host the oracle runs on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def cpu_baseline(wl, logits, x, seconds: float, ffn_weights=None, vsrc=False) -> dict:
    """The oracle, as it stands, timed on the host (single thread), in the
    metric's unit where the path allows it: dispatch + combine tokens/s."""
    import numpy as np

    import oracle

    host = host_description()
    if vsrc:
        passes, t_used = 0, 0.0
        while passes < 2 or t_used < seconds:
            t0 = time.perf_counter()
            idx, w = oracle.route(logits, wl.k)
            v = oracle.vsrc_exchange(x, idx, w, wl.E, wl.R, wl.W)
            oracle.stats(v["expert_counts"], wl.R)
            t_used += time.perf_counter() - t0
            passes += 1
        tokens = wl.T * passes
        sample = (f"{passes} full passes of the {wl.name} workload (T={wl.T}) through the oracle "
                  f"(C steps, numpy block moves): route, per-source dispatch, exchange, regroup, "
                  f"expert, ungroup, exchange back, combine, stats")
    elif ffn_weights is None:
        # routing and the expert rows once, untimed (outside the metric); then
        # whole passes of the oracle's dispatch (counts, offsets, positions,
        # row copy) and combine over all T tokens
        idx, w = oracle.route(logits, wl.k)
        d = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
        out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
        del d
        passes, t_used = 0, 0.0
        while passes < 2 or t_used < seconds:
            t0 = time.perf_counter()
            d = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
            oracle.combine_f64(out, w, d["pos"], wl.T)
            t_used += time.perf_counter() - t0
            passes += 1
            del d
        tokens = wl.T * passes
        sample = (f"{passes} whole passes of the {wl.name} workload (T={wl.T}) through the "
                  f"single-threaded C oracle's dispatch (counts, offsets, positions, row copy) "
                  f"and combine (fp64); routing and expert rows computed once beforehand, "
                  f"untimed")
    else:
        gu, dn = ffn_weights
        tokens, t_used = 0, 0.0
        t = 0
        while t_used < seconds or tokens < 2:
            t0 = time.perf_counter()
            lt = logits[t:t + 1]
            idx, w = oracle.route(lt, wl.k)
            o64, _ = oracle.expert_swiglu_rows(np.repeat(x[t:t + 1], wl.k, 0), idx[0], gu, dn)
            (w[0][:, None] * o64).sum(0)
            t_used += time.perf_counter() - t0
            tokens += 1
            t = (t + 1) % wl.T
        sample = (f"{tokens} tokens of the {wl.name} workload one at a time through the "
                  f"single-threaded C oracle: route, SwiGLU FFN of the k picks (fp64), combine")
    return {"value": round(tokens / t_used, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample}; {t_used:.1f} s on one thread of {host['cpu_model']} "
                      f"({host['nproc']} usable cores)", "host": host}


def wave_sweep(args, wl, moe, torch, np, to_dev, logits_np, x_np) -> dict:
    """T(W) of the wave-pipelined layer: per W dividing L, K steps of
    route+index (fused) -> per wave, a gather dispatch on a copy stream
    overlapped with that wave's experts (the SwiGLU FFN, or the identity-scaled
    experts) on the compute stream -> combine; and the same launches on one
    stream; the two-stream schedule with each wave's completed tokens combined
    in the pipeline (on a third stream, as soon as the wave's experts are
    done); and,
    for reference, the unpipelined copy + expert stage with the same W. Fits
    T(W) = a*W + b + m/W (the page's W*alpha + M/beta + M/(W*beta) plus the
    stages outside the pipeline) to the two-stream times."""
    dev = torch.device("cuda:0")
    T, H, E, k, R = wl.T, wl.H, wl.E, wl.k, wl.R
    L = E // R
    swiglu = wl.expert == "swiglu"
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    logits, x = to_dev(logits_np), to_dev(x_np)
    import synth
    if swiglu:
        gu_np, dn_np = synth.swiglu_weights(wl)
        gu, dn = to_dev(gu_np), to_dev(dn_np)
    side, cstream = torch.cuda.Stream(), torch.cuda.Stream()
    res = {"W": [], "ms_two_streams": [], "ms_one_stream": [], "ms_unpipelined": [],
           "ms_two_streams_wave_combine": []}
    for W in [d for d in range(1, L + 1) if L % d == 0 and args.waves in (None, d)]:
        shape = moe.Shape(T, H, E, k, R, W, tdt)
        buf = moe.alloc_dispatch(shape, dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        wt = torch.empty((T, k), dtype=torch.float32, device=dev)
        eo = torch.empty_like(buf["send_buf"])
        y = torch.empty((T, H), dtype=tdt, device=dev)
        two = torch.empty((W + 1,), dtype=torch.int32, device=dev)
        order = torch.empty((T,), dtype=torch.int32, device=dev)
        wc = dict(topk_w=wt, pos=buf["pos"], token_order=order, token_wave_offsets=two, y=y,
                  stream=cstream)
        if swiglu:
            ws = torch.empty((moe.expert_swiglu_workspace_bytes(shape, wl.I),),
                             dtype=torch.uint8, device=dev)
            chains = moe.Chains(n_events=moe.swiglu_waves_events(W))
        else:
            chains = moe.Chains(n_events=moe.scale_waves_events(W), side=False)

        def step(mode):
            moe.route_index(logits, shape, buf, idx, wt)
            copy = side if mode in ("two", "two_wc") else None
            if mode == "two_wc":
                moe.combine_order(buf["pos"], buf["wave_offsets"], shape, two, order)
                if swiglu:
                    moe.swiglu_waves(x, buf, shape, gu, dn, expert_out=eo, workspace=ws,
                                     copy_stream=copy, chains=chains, combine=wc)
                else:
                    moe.scale_waves(x, buf, shape, expert_out=eo, copy_stream=copy,
                                    chains=chains, combine=wc)
                return
            if mode == "plain":
                moe.dispatch_copy(x, buf["pos"], shape, buf["send_buf"])
                if swiglu:
                    moe.expert_swiglu(buf["send_buf"], buf["expert_offsets"],
                                      buf["expert_counts"], shape, gu, dn, expert_out=eo,
                                      workspace=ws, chains=chains)
                else:
                    moe.expert_scale(buf["send_buf"], buf["expert_offsets"],
                                     buf["expert_counts"], shape, expert_out=eo)
            elif swiglu:
                moe.swiglu_waves(x, buf, shape, gu, dn, expert_out=eo, workspace=ws,
                                 copy_stream=copy, chains=chains)
            else:
                moe.scale_waves(x, buf, shape, expert_out=eo, copy_stream=copy, chains=chains)
            moe.combine(eo, wt, buf["pos"], shape, y=y)

        row = []
        for mode in ("two", "one", "plain", "two_wc"):
            for _ in range(args.warmup):
                step(mode)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                step(mode)
            torch.cuda.synchronize()
            row.append((time.perf_counter() - t0) * 1e3 / args.steps)
        res["W"].append(W)
        res["ms_two_streams"].append(round(row[0], 4))
        res["ms_one_stream"].append(round(row[1], 4))
        res["ms_unpipelined"].append(round(row[2], 4))
        res["ms_two_streams_wave_combine"].append(round(row[3], 4))
        print(f"[bench] W={W}: {row[0]:.4f} ms (two streams), {row[1]:.4f} ms (one), "
              f"{row[2]:.4f} ms (unpipelined), {row[3]:.4f} ms (two streams, per-wave combine)",
              file=sys.stderr, flush=True)
        # the combine forms alone, on the last step's buffers (events on the
        # current stream, median over the steps)
        moe.combine_order(buf["pos"], buf["wave_offsets"], shape, two, order)

        def each():
            for q in range(W):
                moe.combine_waves(eo, wt, buf["pos"], order, two, shape, q, q + 1, y=y)
        alone = {
            "combine": lambda: moe.combine(eo, wt, buf["pos"], shape, y=y),
            "combine_waves_all": lambda: moe.combine_waves(eo, wt, buf["pos"], order, two,
                                                           shape, 0, W, y=y),
            "combine_waves_each": each,
            "combine_order": lambda: moe.combine_order(buf["pos"], buf["wave_offsets"], shape,
                                                       two, order),
        }
        for key, fn in alone.items():
            ts = []
            for i in range(args.warmup + args.steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                if i >= args.warmup:
                    ts.append(a.elapsed_time(b) * 1e3)
            res.setdefault(f"us_{key}", []).append(round(float(np.median(ts)), 1))
        res.setdefault("tokens_per_completion_wave", []).append(
            np.diff(two.cpu().numpy()).tolist())
    Ws = np.array(res["W"], float)
    t = np.array(res["ms_two_streams"]) * 1e-3
    M = T * k * H * wl.elem_bytes  # bytes dispatched per step (the gathered rows)
    fit = None
    if len(Ws) >= 3:  # three parameters
        A = np.stack([Ws, np.ones_like(Ws), 1.0 / Ws], axis=1)
        (a, b, m), *_ = np.linalg.lstsq(A, t, rcond=None)
        fit = {"alpha_us": round(a * 1e6, 3), "const_us": round(b * 1e6, 2),
               "m_us": round(m * 1e6, 2)}
        if a > 0 and m > 0:
            beta = M / m
            w_plan, _ = moe.plan_waves(M, a, beta, L)
            fit.update(beta_GBs=round(beta / 1e9, 1), W_star=round(float(np.sqrt(m / a)), 2),
                       W_plan=w_plan)
    res["fit"] = fit
    res["W_best_measured"] = int(Ws[int(np.argmin(t))])
    res["message_bytes"] = M
    return res


def make_context(wl, moe, torch, np):
    """Device inputs, the shared output buffers and the pre-marshalled C-ABI
    arguments of one workload (everything the mode builders draw on)."""
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    c = SimpleNamespace(wl=wl, moe=moe, torch=torch, dev=dev, tdt=tdt, to_dev=to_dev,
                        T=wl.T, H=wl.H, E=wl.E, k=wl.k, R=wl.R, W=wl.W,
                        swiglu=wl.expert == "swiglu")
    c.logits_np, c.x_np = synth.logits(wl), synth.hidden(wl)
    c.logits, c.x = to_dev(c.logits_np), to_dev(c.x_np)
    c.shape = moe.Shape(c.T, c.H, c.E, c.k, c.R, c.W, tdt)
    c.topk_idx = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
    c.topk_w = torch.empty((c.T, c.k), dtype=torch.float32, device=dev)
    c.y = torch.empty((c.T, c.H), dtype=tdt, device=dev)
    c.stats_raw = torch.empty((moe.STATS_BYTES,), dtype=torch.uint8, device=dev)
    c.ffn_np = synth.swiglu_weights(wl) if c.swiglu else None
    # Pre-marshalled C-ABI calls: the per-step host cost is a few foreign calls.
    c.L = moe.lib()
    c.sh = c.shape.c()
    c.shp = ctypes.byref(c.sh)
    c.P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    c.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return c


# A mode builder returns the step as a list of calls, each (C function,
# arguments, [(stage, kernel) per kernel it launches, in order]), plus what the
# report needs: the algorithmic byte model (evaluated after the timed loops),
# the counts the Dirichlet fit reads, the step's description and extra config.

def path_default(c, args):
    """route + dispatch (index + copy) + experts + combine + stats: separate
    calls (7 kernels a step, 5 when T*k <= 1024) or, with --fused,
    moe_route_dispatch (4 kernels a step when T*k <= 1024, else 5)."""
    moe, L, P, shp, s = c.moe, c.L, c.P, c.shp, c.stream
    buf = moe.alloc_dispatch(c.shape, c.dev)
    expert_out = torch_empty_like(c, buf["send_buf"])
    index_args = (P(buf["expert_counts"]), P(buf["expert_offsets"]), P(buf["rank_counts"]),
                  P(buf["rank_offsets"]), P(buf["wave_offsets"]), P(buf["pos"]),
                  P(buf["row_token"]))
    if c.swiglu:
        gu, dn = c.to_dev(c.ffn_np[0]), c.to_dev(c.ffn_np[1])
        ws = c.torch.empty((moe.expert_swiglu_workspace_bytes(c.shape, c.wl.I),),
                           dtype=c.torch.uint8, device=c.dev)
        chains = moe.Chains()  # the second chain of experts: a side stream and two events
        c.keep = (gu, dn, ws, chains)
        a = (shp, c.wl.I, P(buf["send_buf"]), P(buf["expert_offsets"]), P(buf["expert_counts"]),
             P(gu), P(dn), P(expert_out), P(ws), ws.numel(), s, chains.side_ptr(),
             chains.event_ptr(0), chains.event_ptr(1))
        # the two GEMMs of each chain of experts (the chains run on streams of
        # their own, so the stage is timed as the span of its kernels). The
        # count probe runs before any index stage has filled the tables: empty
        # buckets keep it from touching rows (the launch count does not
        # depend on them).
        buf["expert_counts"].zero_()
        buf["expert_offsets"].zero_()
        nl = launches_of(c, L.moe_expert_swiglu, a)
        if nl < 2 or nl % 2:
            raise RuntimeError(f"moe_expert_swiglu launched {nl} kernels")
        names = ["ffn_gemm_kernel<gate_up>", "ffn_gemm_kernel<down>"] * (nl // 2)
        expert = (L.moe_expert_swiglu, a, [("expert", n) for n in names])
    else:
        expert = (L.moe_expert_scale, (shp, P(buf["send_buf"]), P(buf["expert_offsets"]),
                                       P(buf["expert_counts"]), P(expert_out), s),
                  [("expert", "expert_scale_kernel")])
    # index + copy: one launch when all picks fit one 1024-pick batch (decode)
    one = 0 < c.T * c.k <= 1024 and c.E <= 1024
    if not args.fused:
        calls = [
            (L.moe_route, (P(c.logits), c.T, c.E, c.k, P(c.topk_idx), P(c.topk_w), s),
             [("route", "route_kernel")]),
            (L.moe_dispatch, (shp, P(c.x), P(c.topk_idx), P(buf["send_buf"]), *index_args,
                              P(buf["workspace"]), buf["workspace"].numel(), s),
             [("dispatch", "dispatch_small_kernel")] if one else
             [("dispatch_index", "count_kernel"), ("dispatch_index", "place_kernel"),
              ("dispatch_copy", "copy_kernel")]),
        ]
        desc = ("route+dispatch(" + ("one launch" if one else "count,place,copy")
                + ")+expert+combine+stats")
    else:
        kernels = ([("route", "route_kernel"), ("dispatch", "dispatch_small_kernel(+stats block)")]
                   if one else
                   [("route", "route_count_kernel"), ("dispatch_index", "place_kernel(+stats block)"),
                    ("dispatch_copy", "copy_kernel")])
        calls = [
            (L.moe_route_dispatch, (shp, P(c.logits), P(c.x), P(c.topk_idx), P(c.topk_w),
                                    P(buf["send_buf"]), *index_args, P(c.stats_raw),
                                    P(buf["workspace"]), buf["workspace"].numel(), s), kernels),
        ]
        desc = ("route+dispatch+stats (moe_route_dispatch: "
                + ("two launches" if one else "three launches") + ")+expert+combine")
    calls += [
        expert,
        (L.moe_combine, (shp, P(expert_out), P(c.topk_w), P(buf["pos"]), P(c.y), s),
         [("combine", "combine_kernel")]),
    ]
    if not args.fused:
        calls.append((L.moe_stats, (P(buf["expert_counts"]), c.E, c.R, P(c.stats_raw), s),
                      [("stats", "stats_kernel")]))
    return SimpleNamespace(calls=calls, nbytes=lambda: algorithmic_bytes(c.wl),
                           counts=buf["expert_counts"], desc=desc, config=lambda: {})


def launches_of(c, fn, a) -> int:
    """Kernels one call launches (counted by the library's timing hook)."""
    hipev = HipEvents()
    n = StepRunner.NPAIR
    starts = (ctypes.c_void_p * n)(*[hipev.create() for _ in range(n)])
    stops = (ctypes.c_void_p * n)(*[hipev.create() for _ in range(n)])
    c.L.moe_set_timing_events(starts, stops, n)
    st = fn(*a)
    got = c.L.moe_timed_launches()
    c.L.moe_set_timing_events(None, None, 0)
    if st != 0:
        raise RuntimeError(c.moe.status_string(st))
    c.torch.cuda.synchronize()
    return got


def path_capacity(c, args):
    """Capacity-factor dispatch: route, count/place/copy/pad, experts and
    combine over the padded buckets, stats of the kept counts."""
    moe, L, P, shp, s = c.moe, c.L, c.P, c.shp, c.stream
    cap = moe.expert_capacity(c.k, args.capacity_factor, c.T, c.E)
    cbuf = moe.alloc_dispatch_capacity(c.shape, cap, c.dev)
    ceo = torch_empty_like(c, cbuf["send_buf"])
    rows = cbuf["rows"]
    calls = [
        (L.moe_route, (P(c.logits), c.T, c.E, c.k, P(c.topk_idx), P(c.topk_w), s),
         [("route", "route_kernel")]),
        (L.moe_dispatch_capacity, (
            shp, cap, P(c.x), P(c.topk_idx), P(cbuf["send_buf"]), P(cbuf["kept_counts"]),
            P(cbuf["expert_offsets"]), P(cbuf["rank_counts"]), P(cbuf["rank_offsets"]),
            P(cbuf["wave_offsets"]), P(cbuf["pos"]), P(cbuf["row_token"]),
            P(cbuf["workspace"]), cbuf["workspace"].numel(), s),
         [("dispatch_index", "count_kernel"), ("dispatch_index", "place_kernel(capacity)"),
          ("dispatch_copy", "copy_kernel"), ("dispatch_copy", "pad_kernel")]),
        (L.moe_expert_scale_rows, (shp, rows, P(cbuf["send_buf"]), P(cbuf["expert_offsets"]),
                                   P(cbuf["kept_counts"]), P(ceo), s),
         [("expert", "expert_scale_kernel")]),
        (L.moe_combine_rows, (shp, rows, P(ceo), P(c.topk_w), P(cbuf["pos"]), P(c.y), s),
         [("combine", "combine_kernel")]),
        (L.moe_stats, (P(cbuf["kept_counts"]), c.E, c.R, P(c.stats_raw), s),
         [("stats", "stats_kernel")]),
    ]

    def kept():
        return int(cbuf["kept_counts"].sum().item())

    return SimpleNamespace(
        calls=calls, nbytes=lambda: capacity_bytes(c.wl, cap, kept()),
        counts=cbuf["kept_counts"],
        desc="route+dispatch_capacity(count,place,copy,pad)+expert+combine+stats",
        config=lambda: dict(capacity_factor=args.capacity_factor, capacity=cap,
                            kept_picks=kept(), dropped_picks=c.T * c.k - kept()))


def path_vsrc(c, args):
    """The exchange of R virtual ranks on one device: route, every source's
    dispatch + the count exchange, the all-to-all and the regroup (or, with
    --direct, one copy into the grouped layout), experts, the way back,
    combine, stats."""
    moe, L, P, shp, s = c.moe, c.L, c.P, c.shp, c.stream
    vb = moe.alloc_vsrc(c.shape, c.dev)
    veo = torch_empty_like(c, vb["send_buf"])
    back_recv = torch_empty_like(c, vb["recv_buf"])
    back_send = torch_empty_like(c, vb["send_buf"])
    # the regrouped rows are in plain expert order: the bucket order of W = 1
    c.sh1 = moe.Shape(c.T, c.H, c.E, c.k, c.R, 1, c.tdt).c()
    shp1 = ctypes.byref(c.sh1)
    vws = (P(vb["workspace"]), vb["workspace"].numel())
    ex_tabs = (P(vb["send_offsets"]), P(vb["recv_counts"]), P(vb["recv_offsets"]))
    rg_tabs = (P(vb["src_counts"]), P(vb["recv_offsets"]), P(vb["expert_offsets"]))
    dr_tabs = (P(vb["src_counts"]), P(vb["src_offsets"]), P(vb["expert_offsets"]))
    head = [
        (L.moe_route, (P(c.logits), c.T, c.E, c.k, P(c.topk_idx), P(c.topk_w), s),
         [("route", "route_kernel")]),
        (L.moe_vsrc_dispatch, (
            shp, P(c.x), P(c.topk_idx), P(vb["send_buf"]), P(vb["src_counts"]),
            P(vb["src_offsets"]), P(vb["send_counts"]), P(vb["send_offsets"]),
            P(vb["recv_counts"]), P(vb["recv_offsets"]), P(vb["expert_counts"]),
            P(vb["expert_offsets"]), P(vb["pos"]), *vws, s),
         [("dispatch_index", "count_kernel"), ("dispatch_index", "place_kernel(sources)"),
          ("dispatch_index", "vsrc_plan_kernel"), ("dispatch_copy", "copy_kernel")]),
    ]
    experts = (L.moe_expert_scale_rows, (shp1, c.T * c.k, P(vb["grouped"]),
                                         P(vb["expert_offsets"]), P(vb["expert_counts"]),
                                         P(veo), s),
               [("expert", "expert_scale_kernel")])
    if args.direct:  # one copy each way: send <-> grouped
        middle = [
            (L.moe_vsrc_exchange_direct, (shp, 0, P(vb["send_buf"]), P(vb["grouped"]), *dr_tabs,
                                          *vws, s),
             [("dispatch_index", "regroup_plan_kernel"), ("exchange", "segcopy_kernel<direct>")]),
            experts,
            (L.moe_vsrc_exchange_direct, (shp, 1, P(veo), P(back_send), *dr_tabs, *vws, s),
             [("dispatch_index", "regroup_plan_kernel"), ("exchange", "segcopy_kernel<direct>")]),
        ]
        desc = "direct exchange+expert+direct exchange back"
    else:
        middle = [
            (L.moe_vsrc_exchange, (shp, 0, P(vb["send_buf"]), P(vb["recv_buf"]), *ex_tabs, s),
             [("exchange", "segcopy_kernel<exchange>")]),
            (L.moe_vsrc_regroup, (shp, 0, P(vb["recv_buf"]), P(vb["grouped"]), *rg_tabs, *vws, s),
             [("dispatch_index", "regroup_plan_kernel"), ("regroup", "segcopy_kernel<regroup>")]),
            experts,
            (L.moe_vsrc_regroup, (shp, 1, P(veo), P(back_recv), *rg_tabs, *vws, s),
             [("dispatch_index", "regroup_plan_kernel"), ("regroup", "segcopy_kernel<regroup>")]),
            (L.moe_vsrc_exchange, (shp, 1, P(back_recv), P(back_send), *ex_tabs, s),
             [("exchange", "segcopy_kernel<exchange>")]),
        ]
        desc = "exchange+regroup+expert+ungroup+exchange back"
    tail = [
        (L.moe_combine, (shp, P(back_send), P(c.topk_w), P(vb["pos"]), P(c.y), s),
         [("combine", "combine_kernel")]),
        (L.moe_stats, (P(vb["expert_counts"]), c.E, c.R, P(c.stats_raw), s),
         [("stats", "stats_kernel")]),
    ]
    return SimpleNamespace(
        calls=head + middle + tail,
        nbytes=lambda: vsrc_bytes(c.wl, int(vb["expert_counts"].sum().item())),
        counts=vb["expert_counts"],
        desc="route+vsrc_dispatch(count,place,plan,copy)+" + desc + "+combine+stats",
        config=lambda: {})


def torch_empty_like(c, t):
    return c.torch.empty_like(t)


class StepRunner:
    """Runs the calls of one step; with event arrays, every kernel a call
    launches records start/stop events through the library's timing hook."""

    NPAIR = 8  # event pairs per call (a call launches at most 8 kernels)

    def __init__(self, c, calls, span_stages=()):
        """span_stages: stages whose call runs its kernels on several streams at
        once; such a call is timed from its first kernel's start to its last
        kernel's end instead of by the sum of its kernels."""
        self.c, self.calls, self.span_stages = c, calls, set(span_stages)
        self.hipev = HipEvents()
        self.stages = [st for st in STAGES if any(st == g for cl in calls for g, _ in cl[2])]
        self.kernel_of = {st: "+".join(dict.fromkeys(kn for cl in calls for g, kn in cl[2]
                                                     if g == st)) for st in self.stages}
        self.launches_of = {st: sum(1 for cl in calls for g, _ in cl[2] if g == st)
                            for st in self.stages}
        self.kernel_ms = {}

    def span_stage(self, i):
        """The stage of call i when it is timed as a span, else None."""
        sts = {st for st, _ in self.calls[i][2]}
        return next(iter(sts)) if len(sts) == 1 and sts <= self.span_stages else None

    def step(self, evs=None):
        """One pass of the path; evs[i] = (starts, stops, span) event arrays of
        call i (span: two events recorded on the call's stream around it)."""
        L = self.c.L
        for i, (fn, a, kernels) in enumerate(self.calls):
            span = evs is not None and self.span_stage(i) is not None
            if evs is not None:
                L.moe_set_timing_events(evs[i][0], evs[i][1], self.NPAIR)
            if span:
                self.hipev.record(evs[i][2][0], self.c.stream)
            st = fn(*a)
            if span:
                self.hipev.record(evs[i][2][1], self.c.stream)
            if evs is not None:
                n = L.moe_timed_launches()
                L.moe_set_timing_events(None, None, 0)
                if n != len(kernels):
                    raise RuntimeError(f"call {i} launched {n} kernels, expected {len(kernels)}")
            if st != 0:
                raise RuntimeError(f"call {i}: {self.c.moe.status_string(st)}")

    def new_events(self, n):
        def arr():
            return (ctypes.c_void_p * self.NPAIR)(*[self.hipev.create() for _ in range(self.NPAIR)])
        return [[(arr(), arr(), (self.hipev.create(), self.hipev.create())) for _ in self.calls]
                for _ in range(n)]

    def stage_means(self, evs):
        """Per stage: summed execution time of its kernels, averaged over steps
        (and each kernel's mean time per launch into kernel_ms)."""
        tot = {st: 0.0 for st in self.stages}
        per, n = {}, {}
        self.step_stage_ms = []  # per step: stage -> ms
        for e in evs:
            one = {st: 0.0 for st in self.stages}
            for i, (_, _, kernels) in enumerate(self.calls):
                span = self.span_stage(i)
                for j, (st, kn) in enumerate(kernels):
                    t = self.hipev.ms(e[i][0][j], e[i][1][j])
                    if span is None:
                        tot[st] += t
                        one[st] += t
                    per[kn] = per.get(kn, 0.0) + t
                    n[kn] = n.get(kn, 0) + 1
                if span is not None:
                    t = self.hipev.ms(e[i][2][0], e[i][2][1])
                    tot[span] += t
                    one[span] += t
            self.step_stage_ms.append(one)
        self.kernel_ms = {kn: per[kn] / n[kn] for kn in per}
        return {st: v / len(evs) for st, v in tot.items()}

    @staticmethod
    def median_of(steps, keys) -> float:
        """Median over `steps` (per-step stage -> ms, as stage_means leaves in
        step_stage_ms) of the summed time of `keys` (ms)."""
        v = sorted(sum(one[k] for k in keys) for one in steps)
        m = len(v) // 2
        return v[m] if len(v) % 2 else 0.5 * (v[m - 1] + v[m])

    def graph_wall(self, K):
        """K replays of the step captured in one HIP graph on a side stream."""
        torch = self.c.torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        stream_c = ctypes.c_void_p(side.cuda_stream)
        saved = list(self.calls)
        for i, (fn, a, kn) in enumerate(self.calls):  # rebind the stream argument
            self.calls[i] = (fn, tuple(stream_c if v is self.c.stream else v for v in a), kn)
        with torch.cuda.stream(side):
            self.step()
            torch.cuda.current_stream().synchronize()
            with torch.cuda.graph(g, stream=side):
                self.step()
        torch.cuda.synchronize()
        self.calls[:] = saved
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            g.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0


def plain_rates(torch, dev) -> dict:
    """Reference streaming rates on this machine, with buffers beyond the Infinity
    Cache: the HIP runtime's own 1 GiB device copy (read + write) and torch's
    sum over 1 GiB of fp32 (read-only; its counters also check the scale of the
    read-byte counter on a second kernel of known bytes)."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca.record()
    for _ in range(5):
        dst.copy_(src)
    cb.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9
    del dst
    f = src.view(torch.float32)
    acc = f.sum()
    ca.record()
    for _ in range(5):
        acc = f.sum()
    cb.record()
    torch.cuda.synchronize()
    read_gbs = (1 << 30) * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9
    del acc
    return {"plain_copy_GBs": round(copy_gbs, 1), "plain_read_GBs": round(read_gbs, 1)}


def dirichlet_fit(moe, torch, counts, dev) -> dict:
    """Fitted symmetric Dirichlet alpha of this step's counts: a summary of S
    computed on demand (its own launch), timed apart from the step."""
    alpha_t = torch.empty((1,), dtype=torch.float64, device=dev)
    moe.dirichlet_alpha_device(counts, alpha_t)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record()
    for _ in range(20):
        moe.dirichlet_alpha_device(counts, alpha_t)
    eb.record()
    torch.cuda.synchronize()
    return {"value": float(alpha_t.item()), "us": round(ea.elapsed_time(eb) * 1e3 / 20, 2),
            "kernel": "dirichlet_alpha_kernel", "in_step": False}


def wave_sweep_result(args, wl, moe, torch, np, c) -> dict:
    ws_res = wave_sweep(args, wl, moe, torch, np, c.to_dev, c.logits_np, c.x_np)
    best = ws_res["W"].index(ws_res["W_best_measured"])
    ms = ws_res["ms_two_streams"][best]
    swiglu = wl.expert == "swiglu"
    return {
        "metric": METRIC, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded logits and hidden states"
                + ("; random-init SwiGLU expert weights)" if swiglu else "; identity-scaled experts)"),
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "k": wl.k,
                   "virtual_ranks": wl.R, "waves": ws_res["W_best_measured"],
                   **({"I": wl.I} if swiglu else {}), "expert": wl.expert,
                   "step": "route+index (moe_route_index) + per wave: gather dispatch (copy "
                           "stream) -> experts (compute stream) + combine; value = whole-step "
                           "tokens/s at the best W"},
        "wave_sweep": ws_res,
    }


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path, so --gpus "
              f"{args.gpus} (WORLD_SIZE={world}) is not supported; run with --gpus 1.",
              file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import combine_moe_route_03_amd as moe
    import synth

    wl = synth.WORKLOADS[args.workload]
    swiglu = wl.expert == "swiglu"
    if (args.capacity_factor is not None or args.vsrc) and swiglu:
        print("--capacity-factor and --vsrc run the identity-scaled experts", file=sys.stderr)
        return 2
    if args.capacity_factor is not None and args.vsrc:
        print("--vsrc runs without a capacity", file=sys.stderr)
        return 2
    print(f"[bench] workload {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} W={wl.W} "
          f"{wl.dtype} expert={wl.expert}", file=sys.stderr, flush=True)
    c = make_context(wl, moe, torch, np)
    if args.wave_sweep:
        print(json.dumps(wave_sweep_result(args, wl, moe, torch, np, c)), flush=True)
        return 0
    if args.capacity_factor is not None:
        path = path_capacity(c, args)
    elif args.vsrc:
        path = path_vsrc(c, args)
    else:
        path = path_default(c, args)
    run = StepRunner(c, path.calls, span_stages=("expert",) if swiglu else ())
    T, K = wl.T, args.steps

    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()

    # ---- timed region 1: K plain steps -> value
    t0 = time.perf_counter()
    for _ in range(K):
        run.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {K} timed steps in {wall * 1e3:.2f} ms", file=sys.stderr, flush=True)

    # ---- timed region 2: K instrumented steps -> per-stage kernel times
    evs = run.new_events(K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run.step(evs[i])
    torch.cuda.synchronize()
    wall_instr = time.perf_counter() - t0
    stage_ms = run.stage_means(evs)
    warm_steps = list(run.step_stage_ms)
    kernel_us = {kn: round(v * 1e3, 2) for kn, v in run.kernel_ms.items()}
    nbytes = path.nbytes()

    # ---- timed region 3: only the calls whose kernels all belong to dispatch
    # or combine, K times -> their wall clock (launch gaps included)
    dc_calls = [cl for cl in path.calls if cl[2] and all(st in DC_STAGES for st, _ in cl[2])]
    dc_wall = None
    if dc_calls:
        dc_run = StepRunner(c, dc_calls)
        for _ in range(max(1, args.warmup // 2)):
            dc_run.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            dc_run.step()
        torch.cuda.synchronize()
        dc_wall = time.perf_counter() - t0

    graph_wall = run.graph_wall(K) if args.graph else None
    rates = plain_rates(torch, c.dev)

    cold_ms = None
    if not args.no_cold:
        # the same instrumented step after evicting the 256 MB Infinity Cache
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=c.dev)
        Kc = max(5, min(K, 50))
        cevs = run.new_events(Kc)
        for i in range(Kc):
            flush.fill_(i & 0xFF)
            run.step(cevs[i])
        torch.cuda.synchronize()
        cold_ms = run.stage_means(cevs)
        cold_steps = list(run.step_stage_ms)
        del flush

    alpha_fit = dirichlet_fit(moe, torch, path.counts, c.dev)
    stages, kernel_of, launches_of = run.stages, run.kernel_of, run.launches_of

    def gbs(name, ms):
        return nbytes[name] / (ms * 1e-3) / 1e9

    def stage_report(ms):
        rep = {}
        for n in stages:
            rep[n] = {"us": round(ms[n] * 1e3, 2), "GB/s": round(gbs(n, ms[n]), 1),
                      "frac_hbm_peak": round(gbs(n, ms[n]) / HBM_PEAK_GBS, 4),
                      "kernels": kernel_of[n]}
        if swiglu:
            tf = ffn_flops(wl) / (ms["expert"] * 1e-3) / 1e12
            rep["expert"]["TFLOP/s"] = round(tf, 1)
            rep["expert"]["frac_mfma_bf16_peak"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        return rep

    dc_keys = tuple(n for n in DC_STAGES if n in stage_ms)
    dc_ms = sum(stage_ms[n] for n in dc_keys)
    dc_med = StepRunner.median_of(warm_steps, dc_keys)
    dc_bytes = sum(nbytes[n] for n in dc_keys)

    def roofline_hbm(n, ms):
        # per launch: a stage may launch its kernel more than once a step (the
        # exchange and the regroup run forward and back), bytes and time both scale
        nl = launches_of[n]
        return {"bound": "hbm", "kernel": kernel_of[n], "achieved": round(gbs(n, ms[n]), 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs(n, ms[n]) / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic(wl.name, kernel_of[n]),
                "bytes_per_launch": nbytes[n] // nl, "launches_per_step": nl,
                "avg_us": round(ms[n] * 1e3 / nl, 2)}

    # The dominant single-kernel stage of the metric's region (the row copies;
    # the index stage is a few small kernels): the headline roofline.
    single = [n for n in ("dispatch", "dispatch_copy", "exchange", "regroup", "combine")
              if n in stages]
    dom = max(single, key=lambda n: stage_ms[n])
    roofline = roofline_hbm(dom, stage_ms)
    # The expert stage sits between dispatch and combine but outside the metric.
    if swiglu:
        tf = ffn_flops(wl) / (stage_ms["expert"] * 1e-3) / 1e12
        expert_roofline = {"bound": "mfma", "kernel": kernel_of["expert"],
                           "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                           "traffic": stored_traffic(wl.name, kernel_of["expert"]),
                           "flops_per_call": ffn_flops(wl),
                           "avg_us": round(stage_ms["expert"] * 1e3, 2)}
    else:
        expert_roofline = roofline_hbm("expert", stage_ms)

    result = {
        "metric": METRIC,
        "value": round(T / (dc_med * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded logits and hidden states"
                + ("; random-init SwiGLU expert weights)" if swiglu else "; identity-scaled experts)"),
        "config": {"workload": wl.name, "T": T, "H": wl.H, "E": wl.E, "k": wl.k,
                   "virtual_ranks": wl.R, "waves": wl.W, "routing": wl.routing,
                   "expert": wl.expert, "step": path.desc,
                   "kernels_per_step": sum(len(cl[2]) for cl in path.calls),
                   **({"I": wl.I} if swiglu else {}), **path.config()},
        "step_tokens_per_s": round(T * K / wall, 1),
        "dispatch_combine": {
            "median_us": round(dc_med * 1e3, 2),
            "mean_us": round(dc_ms * 1e3, 2),
            "tokens_per_s": round(T / (dc_med * 1e-3), 1),
            "GB/s": round(dc_bytes / (dc_med * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(dc_bytes / (dc_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": dc_bytes,
            "kernels": "+".join(kernel_of[n] for n in dc_keys),
            "timing": "median over the instrumented steps of the summed kernel execution times",
            **({"wall_us": round(dc_wall * 1e6 / K, 2),
                "wall_calls": "+".join(cl[0].__name__ for cl in dc_calls),
                "wall_frac_hbm_peak": round(
                    sum(nbytes[st] for st in {g for cl in dc_calls for g, _ in cl[2]})
                    / (dc_wall / K) / 1e9 / HBM_PEAK_GBS, 4)}
               if dc_wall is not None else {}),
        },
        "roofline": roofline,
        "expert_roofline": expert_roofline,
        "stages": stage_report(stage_ms),
        "kernel_us_per_launch": kernel_us,
        "stage_timing": "sum of the execution times of each stage's kernels, from start/stop "
                        "events recorded by the library's extended launches (instrumented loop "
                        f"of {K} steps, {wall_instr * 1e3 / K:.4f} ms/step wall)",
        **rates,
        "dirichlet_alpha": alpha_fit,
    }
    if graph_wall is not None:
        result["graph_replay"] = {"ms_per_step": round(graph_wall * 1e3 / K, 4),
                                  "tokens_per_s": round(T * K / graph_wall, 1)}
    if cold_ms is not None:
        cdc = StepRunner.median_of(cold_steps, dc_keys)
        result["cold_cache"] = {
            "stages": stage_report(cold_ms),
            "dispatch_combine": {"median_us": round(cdc * 1e3, 2),
                                 "mean_us": round(sum(cold_ms[n] for n in dc_keys) * 1e3, 2),
                                 "tokens_per_s": round(T / (cdc * 1e-3), 1),
                                 "GB/s": round(dc_bytes / (cdc * 1e-3) / 1e9, 1),
                                 "frac_hbm_peak": round(dc_bytes / (cdc * 1e-3) / 1e9
                                                        / HBM_PEAK_GBS, 4)}}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, c.logits_np, c.x_np, args.cpu_seconds, c.ffn_np,
                                              vsrc=args.vsrc)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

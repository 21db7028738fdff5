#!/usr/bin/env python3
"""Benchmark of the one-GPU MoE routing path on an MI355X.

One step = the whole path on one batch of synthetic input, inputs already in
HBM: route (top-k gating) -> dispatch index (counts, offsets, positions) ->
dispatch copy (permute into the send buffer) -> identity-scaled experts ->
combine -> skew statistics. Every step runs in the library's HIP kernels on
torch's current stream; torch only provides memory, the stream and events.

Prints ONE JSON line. `value` is whole-step tokens/s over the K timed steps
(wall clock, bracketed by synchronisations). Per-stage kernel times come from
HIP events recorded on the launch stream inside the same timed region; the
dominant kernel's algorithmic bytes / its average duration gives `roofline`.
A second, untimed-for-`value` loop repeats the steps after evicting the 256 MB
Infinity Cache (512 MiB scratch write) to report cold-cache stage times.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/sec and achieved HBM GB/s (% of peak) on 1 MI355X"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
STAGES = ("route", "dispatch_index", "dispatch_copy", "expert", "combine", "stats")
# Stages that are exactly one kernel launch (roofline candidates).
SINGLE_KERNEL = {"route": "route_kernel", "dispatch_copy": "copy_kernel",
                 "expert": "expert_scale_kernel", "combine": "combine_kernel",
                 "stats": "stats_kernel"}


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded (same soname)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(out), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return out.value


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="zipf")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-evicted loop")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--graph", action="store_true",
                    help="also time K steps replayed from one captured HIP graph")
    return ap.parse_args()


def algorithmic_bytes(wl) -> dict:
    """Minimum HBM bytes each stage must move (per launch)."""
    T, H, E, k, b = wl.T, wl.H, wl.E, wl.k, wl.elem_bytes
    return {
        "route": T * E * 4 + T * k * 8,                  # logits in; idx + w out
        "dispatch_index": 12 * T * k,                    # idx in; pos + row_token out
        "dispatch_copy": T * H * b + T * k * H * b + 4 * T * k,  # x once, k copies, pos
        "expert": 2 * T * k * H * b,                     # send rows in, expert rows out
        "combine": T * k * H * b + 8 * T * k + T * H * b,  # k rows, w + pos in; y out
        "stats": 4 * E,
    }


def cpu_baseline(wl, logits, x, seconds: float) -> dict:
    """The oracle, as it stands, timed on the host on whole passes of the workload."""
    import oracle

    passes, t_used = 0, 0.0
    while passes < 2 or t_used < seconds:
        t0 = time.perf_counter()
        idx, w = oracle.route(logits, wl.k)
        d = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
        out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
        oracle.combine_f64(out, w, d["pos"], wl.T)
        oracle.stats(d["expert_counts"], wl.R)
        t_used += time.perf_counter() - t0
        passes += 1
    return {"value": round(wl.T * passes / t_used, 1), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{passes} full passes of the {wl.name} workload (T={wl.T}) through the "
                      f"single-threaded C oracle: route, dispatch, expert, combine (fp64), stats; "
                      f"{t_used:.1f} s on {platform.processor() or platform.machine()}"}


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
    if wl.expert != "scale":
        wl = wl.with_(expert="scale")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    T, H, E, k, R, W = wl.T, wl.H, wl.E, wl.k, wl.R, wl.W
    print(f"[bench] workload {wl.name}: T={T} H={H} E={E} k={k} R={R} W={W} {wl.dtype}",
          file=sys.stderr, flush=True)

    logits_np, x_np = synth.logits(wl), synth.hidden(wl)
    logits = torch.from_numpy(logits_np).to(dev)
    x = (torch.from_numpy(x_np).to(dev) if wl.dtype == "f32"
         else torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16))
    shape = moe.Shape(T, H, E, k, R, W, tdt)
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    buf = moe.alloc_dispatch(shape, dev)
    expert_out = torch.empty_like(buf["send_buf"])
    y = torch.empty((T, H), dtype=tdt, device=dev)
    stats_raw = torch.empty((moe.STATS_BYTES,), dtype=torch.uint8, device=dev)

    # Pre-marshalled C-ABI calls: the per-step host cost is six foreign calls.
    L = moe.lib()
    sh = shape.c()
    shp = ctypes.byref(sh)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = {
        "route": (L.moe_route, (P(logits), T, E, k, P(topk_idx), P(topk_w), stream)),
        "dispatch_index": (L.moe_dispatch_index, (
            shp, P(topk_idx), P(buf["expert_counts"]), P(buf["expert_offsets"]),
            P(buf["rank_counts"]), P(buf["rank_offsets"]), P(buf["wave_offsets"]), P(buf["pos"]),
            P(buf["row_token"]), P(buf["workspace"]), buf["workspace"].numel(), stream)),
        "dispatch_copy": (L.moe_dispatch_copy, (shp, P(x), P(buf["pos"]), P(buf["send_buf"]),
                                                stream)),
        "expert": (L.moe_expert_scale, (shp, P(buf["send_buf"]), P(buf["expert_offsets"]),
                                        P(buf["expert_counts"]), P(expert_out), stream)),
        "combine": (L.moe_combine, (shp, P(expert_out), P(topk_w), P(buf["pos"]), P(y), stream)),
        "stats": (L.moe_stats, (P(buf["expert_counts"]), E, R, P(stats_raw), stream)),
    }

    hipev = HipEvents()
    set_events = L.moe_set_timing_events

    def step(kev=None, iev=None):
        """One pass of the path. kev[name] = (start, stop) raw events filled by the
        library's extended launches (kernel execution time); iev = torch events
        around the two-kernel index stage."""
        for name in STAGES:
            fn, a = calls[name]
            if name == "dispatch_index" and iev is not None:
                iev[0].record()
            if kev is not None and name in kev:
                set_events(*kev[name])
            st = fn(*a)
            if kev is not None and name in kev:
                set_events(None, None)
            if name == "dispatch_index" and iev is not None:
                iev[1].record()
            if st != 0:
                raise RuntimeError(f"{name}: {moe.status_string(st)}")

    def timed_events(n):
        kev = [{nm: (hipev.create(), hipev.create()) for nm in SINGLE_KERNEL} for _ in range(n)]
        iev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        return kev, iev

    def stage_means(kev, iev):
        out = {nm: float(np.mean([hipev.ms(*kv[nm]) for kv in kev])) for nm in SINGLE_KERNEL}
        out["dispatch_index"] = float(np.mean([a.elapsed_time(b) for a, b in iev]))
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    kev, iev = timed_events(K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(kev[i], iev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {K} timed steps in {wall * 1e3:.2f} ms", file=sys.stderr, flush=True)
    stage_ms = stage_means(kev, iev)
    nbytes = algorithmic_bytes(wl)

    # Same steps without any timing events (host launch cost only).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step()
    torch.cuda.synchronize()
    wall_plain = time.perf_counter() - t0

    graph_wall = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stream_c = ctypes.c_void_p(side.cuda_stream)
            for nm in calls:  # rebind the stream argument to the capture stream
                fn, a = calls[nm]
                calls[nm] = (fn, tuple(stream_c if x is stream else x for x in a))
            step()
            torch.cuda.current_stream().synchronize()
            with torch.cuda.graph(g, stream=side):
                step()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            g.replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t0
        for nm in calls:
            fn, a = calls[nm]
            calls[nm] = (fn, tuple(stream if x is stream_c else x for x in a))

    # Plain device copy of 1 GiB (beyond the Infinity Cache): the bandwidth a
    # trivial streaming kernel reaches on this machine.
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
    del src, dst

    cold_ms = None
    if not args.no_cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        Kc = max(5, min(K, 50))
        ckev, ciev = timed_events(Kc)
        for i in range(Kc):
            flush.fill_(i & 0xFF)
            step(ckev[i], ciev[i])
        torch.cuda.synchronize()
        cold_ms = stage_means(ckev, ciev)
        del flush

    dom = max(SINGLE_KERNEL, key=lambda n: stage_ms[n])
    dom_gbs = nbytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    dc_ms = stage_ms["dispatch_index"] + stage_ms["dispatch_copy"] + stage_ms["combine"]
    dc_bytes = nbytes["dispatch_index"] + nbytes["dispatch_copy"] + nbytes["combine"]

    def stage_report(ms):
        return {n: {"us": round(ms[n] * 1e3, 2),
                    "GB/s": round(nbytes[n] / (ms[n] * 1e-3) / 1e9, 1),
                    "frac_hbm_peak": round(nbytes[n] / (ms[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                for n in STAGES}

    result = {
        "metric": METRIC,
        "value": round(T * K / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded logits and hidden states; identity-scaled experts)",
        "config": {"workload": wl.name, "T": T, "H": H, "E": E, "k": k, "virtual_ranks": R,
                   "waves": W, "routing": wl.routing,
                   "step": "route+dispatch_index+dispatch_copy+expert+combine+stats"},
        "dispatch_combine": {
            "us": round(dc_ms * 1e3, 2),
            "tokens_per_s": round(T / (dc_ms * 1e-3), 1),
            "GB/s": round(dc_bytes / (dc_ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(dc_bytes / (dc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": dc_bytes,
        },
        "roofline": {"bound": "hbm", "kernel": SINGLE_KERNEL[dom], "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": nbytes[dom], "avg_us": round(stage_ms[dom] * 1e3, 2)},
        "stages": stage_report(stage_ms),
        "wall_ms_per_step_without_timing_events": round(wall_plain * 1e3 / K, 4),
        "plain_copy_GBs": round(copy_gbs, 1),
        "stage_timing": "kernel start/stop events from the library's extended launches; "
                        "dispatch_index = torch events around its two kernels",
    }
    if graph_wall is not None:
        result["graph_replay"] = {"ms_per_step": round(graph_wall * 1e3 / K, 4),
                                  "tokens_per_s": round(T * K / graph_wall, 1)}
    if cold_ms is not None:
        cdc = cold_ms["dispatch_index"] + cold_ms["dispatch_copy"] + cold_ms["combine"]
        result["cold_cache"] = {
            "stages": stage_report(cold_ms),
            "dispatch_combine": {"us": round(cdc * 1e3, 2),
                                 "tokens_per_s": round(T / (cdc * 1e-3), 1),
                                 "GB/s": round(dc_bytes / (cdc * 1e-3) / 1e9, 1),
                                 "frac_hbm_peak": round(dc_bytes / (cdc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, logits_np, x_np, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

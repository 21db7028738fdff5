"""Python binding of libmoe_route.so, the gfx950 MoE routing / dispatch / combine library.

Argument marshalling only: every step runs in the library's HIP kernels on the
caller's current torch stream. torch provides device memory and the stream;
outputs are allocated with torch when the caller does not pass them. The
library must be built (``__graft_entry__.build()``); importing the functions
without it raises, there is no fallback.

Entry points mirror include/moe_route.h: ``route``, ``dispatch_index``,
``route_index``, ``dispatch_copy``, ``dispatch``, ``dispatch_capacity``,
``expert_scale``, ``expert_scale_rows``, ``expert_swiglu``, ``combine``,
``combine_rows``, ``stats``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ROUTE_LIB names another build of the same library (the host-sanitized
# build the CPU sanitizer run loads); there is no fallback when it is missing.
LIB_PATH = os.environ.get("MOE_ROUTE_LIB") or os.path.join(_HERE, "libmoe_route.so")

MOE_F32, MOE_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
_CODE_DTYPE = {v: k for k, v in _DTYPE_CODE.items()}


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("R", ctypes.c_int32), ("W", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class MoeStats(ctypes.Structure):
    _fields_ = [("expert_max_over_mean", ctypes.c_double), ("expert_gini", ctypes.c_double),
                ("rank_max_over_mean", ctypes.c_double), ("rank_gini", ctypes.c_double),
                ("total", ctypes.c_int64), ("expert_max", ctypes.c_int32),
                ("expert_min", ctypes.c_int32), ("rank_max", ctypes.c_int32),
                ("rank_min", ctypes.c_int32)]


STATS_BYTES = ctypes.sizeof(MoeStats)

# Every extern "C" function of include/moe_route.h with its ctypes signature.
_vp, _i32, _i32p, _f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
_shp = ctypes.POINTER(MoeShape)
SIGNATURES = {
    "moe_route": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "moe_dispatch_workspace_bytes": ([_shp], ctypes.c_size_t),
    "moe_dispatch_index": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                            _vp], ctypes.c_int),
    "moe_route_index": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         ctypes.c_size_t, _vp], ctypes.c_int),
    "moe_dispatch_copy": ([_shp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_route_dispatch": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "moe_dispatch": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                      ctypes.c_size_t, _vp], ctypes.c_int),
    "moe_dispatch_noalloc": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
                             ctypes.c_int),
    "moe_noalloc_scratch_bytes": ([], ctypes.c_size_t),
    "moe_expert_scale": ([_shp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_expert_scale_rows": ([_shp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_expert_capacity": ([_i32, ctypes.c_double, _i32, _i32], ctypes.c_int32),
    "moe_wave_time": ([ctypes.c_double, ctypes.c_double, ctypes.c_double, _i32], ctypes.c_double),
    "moe_plan_waves": ([ctypes.c_double, ctypes.c_double, ctypes.c_double, _i32,
                        ctypes.POINTER(ctypes.c_double)], ctypes.c_int32),
    "moe_link_p95": ([ctypes.c_double, ctypes.c_double, _i32], ctypes.c_double),
    "moe_dispatch_capacity": ([_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               ctypes.c_size_t, _vp], ctypes.c_int),
    "moe_combine_rows": ([_shp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_swiglu_waves": ([_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          ctypes.c_size_t, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _i32], ctypes.c_int),
    "moe_swiglu_waves_events": ([_i32], ctypes.c_int32),
    "moe_scale_waves": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _vp, _vp, _vp, _i32], ctypes.c_int),
    "moe_scale_waves_events": ([_i32], ctypes.c_int32),
    "moe_combine_order": ([_shp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "moe_combine_order_workspace_bytes": ([_shp], ctypes.c_size_t),
    "moe_combine_waves": ([_shp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "moe_vsrc_workspace_bytes": ([_shp], ctypes.c_size_t),
    "moe_vsrc_dispatch": ([_shp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           ctypes.c_size_t, _vp], ctypes.c_int),
    "moe_vsrc_exchange_direct": ([_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
                                 ctypes.c_int),
    "moe_vsrc_exchange": ([_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_vsrc_regroup": ([_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
                         ctypes.c_int),
    "moe_expert_swiglu_workspace_bytes": ([_shp, _i32], ctypes.c_size_t),
    "moe_expert_swiglu": ([_shp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp,
                           _vp, _vp, _vp], ctypes.c_int),
    "moe_combine": ([_shp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe_stats": ([_vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "moe_dirichlet_alpha": ([_vp, _i32, _vp, _vp], ctypes.c_int),
    "moe_set_timing_events": ([_vp, _vp, _i32], ctypes.c_int),
    "moe_timed_launches": ([], ctypes.c_int),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_route.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MoeError(status, where)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe_route must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


@dataclass(frozen=True)
class Shape:
    T: int
    H: int
    E: int
    k: int
    R: int
    W: int
    dtype: torch.dtype

    def c(self) -> MoeShape:
        return MoeShape(self.T, self.H, self.E, self.k, self.R, self.W, _DTYPE_CODE[self.dtype])

    @property
    def L(self) -> int:
        return self.E // self.R


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


class Chains:
    """Caller-owned stream resources of the FFN entry points: a side stream for
    the second chain of experts (None: one chain) and n_events events (torch
    objects; the library keeps none of them). Create it before capturing a
    graph that uses it: the event handles are materialised here by one record
    on the side stream (or the current stream)."""

    def __init__(self, n_events: int = 2, side: bool = True, device=None):
        self.stream = torch.cuda.Stream(device=device) if side else None
        self.events = [torch.cuda.Event() for _ in range(n_events)]
        where = self.stream if self.stream is not None else torch.cuda.current_stream(device)
        for e in self.events:
            e.record(where)
        self._handles = (ctypes.c_void_p * max(n_events, 1))(
            *[ctypes.c_void_p(e.cuda_event) for e in self.events])

    def side_ptr(self) -> ctypes.c_void_p | None:
        return None if self.stream is None else ctypes.c_void_p(self.stream.cuda_stream)

    def event_ptr(self, i: int) -> ctypes.c_void_p:
        return ctypes.c_void_p(self.events[i].cuda_event)

    def event_array(self):
        return self._handles


def swiglu_waves_events(W: int) -> int:
    return int(lib().moe_swiglu_waves_events(W))


def scale_waves_events(W: int) -> int:
    return int(lib().moe_scale_waves_events(W))


# ----------------------------------------------------------------------- route

def route(logits: torch.Tensor, k: int, topk_idx: torch.Tensor | None = None,
          topk_w: torch.Tensor | None = None):
    """Top-k gating: (topk_idx int32 [T,k], topk_w float32 [T,k])."""
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    dev = logits.device
    topk_idx = _empty((T, k), torch.int32, dev) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, dev) if topk_w is None else topk_w
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w), _stream()),
           "moe_route")
    return topk_idx, topk_w


# -------------------------------------------------------------------- dispatch

def dispatch_workspace_bytes(shape: Shape) -> int:
    sh = shape.c()
    return int(lib().moe_dispatch_workspace_bytes(ctypes.byref(sh)))


def alloc_dispatch(shape: Shape, device) -> dict:
    """Output and workspace buffers of one dispatch call for this shape."""
    T, k, E, R, W, H = shape.T, shape.k, shape.E, shape.R, shape.W, shape.H
    i32 = torch.int32
    return dict(
        send_buf=_empty((T * k, H), shape.dtype, device),
        expert_counts=_empty((E,), i32, device), expert_offsets=_empty((E,), i32, device),
        rank_counts=_empty((W * R,), i32, device), rank_offsets=_empty((W * R,), i32, device),
        wave_offsets=_empty((W + 1,), i32, device), pos=_empty((T, k), i32, device),
        row_token=_empty((T * k,), i32, device),
        workspace=_empty((max(dispatch_workspace_bytes(shape), 1),), torch.uint8, device))


def dispatch_index(topk_idx: torch.Tensor, shape: Shape, out: dict):
    """Counts, offsets and positions into the buffers of `out` (see alloc_dispatch)."""
    sh = shape.c()
    _check(lib().moe_dispatch_index(
        ctypes.byref(sh), _ptr(topk_idx), _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]), _ptr(out["wave_offsets"]),
        _ptr(out["pos"]), _ptr(out["row_token"]), _ptr(out["workspace"]),
        out["workspace"].numel(), _stream()), "moe_dispatch_index")
    return out


def route_index(logits: torch.Tensor, shape: Shape, out: dict, topk_idx: torch.Tensor,
                topk_w: torch.Tensor, stats_out: torch.Tensor | None = None) -> dict:
    """Routing + counts, offsets, positions (+ statistics into the raw device
    struct `stats_out` when given) in two launches; buffers as alloc_dispatch."""
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    sh = shape.c()
    _check(lib().moe_route_index(
        ctypes.byref(sh), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(out["expert_counts"]),
        _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]),
        _ptr(out["wave_offsets"]), _ptr(out["pos"]), _ptr(out["row_token"]), _ptr(stats_out),
        _ptr(out["workspace"]), out["workspace"].numel(), _stream()), "moe_route_index")
    return out


def route_dispatch(logits: torch.Tensor, x: torch.Tensor, shape: Shape, out: dict,
                   topk_idx: torch.Tensor, topk_w: torch.Tensor,
                   stats: torch.Tensor | None = None) -> dict:
    """Routing, index stage, optional statistics and the dispatch copy (one
    launch when T*k <= 1024) into topk_idx / topk_w and the buffers of `out`."""
    sh = shape.c()
    _check(lib().moe_route_dispatch(
        ctypes.byref(sh), _ptr(logits), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
        _ptr(out["send_buf"]), _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]), _ptr(out["wave_offsets"]),
        _ptr(out["pos"]), _ptr(out["row_token"]), _ptr(stats), _ptr(out["workspace"]),
        out["workspace"].numel(), _stream()), "moe_route_dispatch")
    return out


def dispatch_copy(x: torch.Tensor, pos: torch.Tensor, shape: Shape, send_buf: torch.Tensor):
    sh = shape.c()
    _check(lib().moe_dispatch_copy(ctypes.byref(sh), _ptr(x), _ptr(pos), _ptr(send_buf),
                                   _stream()), "moe_dispatch_copy")
    return send_buf


def dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, R: int, W: int,
             out: dict | None = None) -> dict:
    """Counts, offsets, positions and the permuted send buffer (one call)."""
    T, H = x.shape
    k = topk_idx.shape[1]
    shape = Shape(T, H, E, k, R, W, x.dtype)
    out = alloc_dispatch(shape, x.device) if out is None else out
    sh = shape.c()
    _check(lib().moe_dispatch(
        ctypes.byref(sh), _ptr(x), _ptr(topk_idx), _ptr(out["send_buf"]),
        _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]),
        _ptr(out["rank_offsets"]), _ptr(out["wave_offsets"]), _ptr(out["pos"]),
        _ptr(out["row_token"]), _ptr(out["workspace"]), out["workspace"].numel(), _stream()),
        "moe_dispatch")
    return out


def dispatch_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, shape: Shape, out: dict) -> dict:
    """moe_dispatch without a workspace: the library's static per-device array
    holds the index stage's histograms. `out` holds the output buffers (its
    "workspace" entry, if any, is not used). Calls overlapping on one device
    race on that array."""
    sh = shape.c()
    _check(lib().moe_dispatch_noalloc(
        ctypes.byref(sh), _ptr(x), _ptr(topk_idx), _ptr(out["send_buf"]),
        _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]),
        _ptr(out["rank_offsets"]), _ptr(out["wave_offsets"]), _ptr(out["pos"]),
        _ptr(out["row_token"]), _stream()), "moe_dispatch_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().moe_noalloc_scratch_bytes())


# ------------------------------------------------------- capacity-factor path

def expert_capacity(k: int, f: float, T: int, E: int) -> int:
    """Rows per expert for capacity factor f (ceil(k*f*T/E)); -1 if invalid."""
    return int(lib().moe_expert_capacity(k, f, T, E))


def wave_time(message_bytes: float, alpha_s: float, beta: float, W: int) -> float:
    """T(W) = W alpha + M/beta + M/(W beta) of the wave-scheduled exchange."""
    return float(lib().moe_wave_time(message_bytes, alpha_s, beta, W))


def plan_waves(message_bytes: float, alpha_s: float, beta: float, L: int):
    """(W, T(W)): the divisor of L with the smallest modelled exchange time."""
    t = ctypes.c_double()
    W = int(lib().moe_plan_waves(message_bytes, alpha_s, beta, L, ctypes.byref(t)))
    return W, t.value


def link_p95(mean_bytes: float, tokens: float, destinations: int) -> float:
    return float(lib().moe_link_p95(mean_bytes, tokens, destinations))


def alloc_dispatch_capacity(shape: Shape, capacity: int, device) -> dict:
    E, R, W, H, T, k = shape.E, shape.R, shape.W, shape.H, shape.T, shape.k
    i32 = torch.int32
    rows = E * capacity
    return dict(
        send_buf=_empty((rows, H), shape.dtype, device), kept_counts=_empty((E,), i32, device),
        expert_offsets=_empty((E,), i32, device), rank_counts=_empty((W * R,), i32, device),
        rank_offsets=_empty((W * R,), i32, device), wave_offsets=_empty((W + 1,), i32, device),
        pos=_empty((T, k), i32, device), row_token=_empty((max(rows, 1),), i32, device),
        workspace=_empty((max(dispatch_workspace_bytes(shape), 1),), torch.uint8, device),
        rows=rows)


def dispatch_capacity(x: torch.Tensor, topk_idx: torch.Tensor, E: int, R: int, W: int,
                      capacity: int, out: dict | None = None) -> dict:
    """Capacity-factor dispatch: buckets of exactly `capacity` rows, overflow
    dropped in token order, zero padding (four launches)."""
    T, H = x.shape
    k = topk_idx.shape[1]
    shape = Shape(T, H, E, k, R, W, x.dtype)
    out = alloc_dispatch_capacity(shape, capacity, x.device) if out is None else out
    sh = shape.c()
    _check(lib().moe_dispatch_capacity(
        ctypes.byref(sh), capacity, _ptr(x), _ptr(topk_idx), _ptr(out["send_buf"]),
        _ptr(out["kept_counts"]), _ptr(out["expert_offsets"]), _ptr(out["rank_counts"]),
        _ptr(out["rank_offsets"]), _ptr(out["wave_offsets"]), _ptr(out["pos"]),
        _ptr(out["row_token"]), _ptr(out["workspace"]), out["workspace"].numel(), _stream()),
        "moe_dispatch_capacity")
    return out


# ------------------------------------------------ virtual-source exchange

def vsrc_workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_vsrc_workspace_bytes(ctypes.byref(shape.c())))


def alloc_vsrc(shape: Shape, device) -> dict:
    """Buffers of the emulated exchange: three row buffers of T*k rows (send,
    recv, grouped) and the count tables."""
    E, R, W, H, T, k = shape.E, shape.R, shape.W, shape.H, shape.T, shape.k
    i32 = torch.int32
    rows = T * k
    return dict(
        send_buf=_empty((rows, H), shape.dtype, device), recv_buf=_empty((rows, H), shape.dtype, device),
        grouped=_empty((rows, H), shape.dtype, device), src_counts=_empty((R, E), i32, device),
        src_offsets=_empty((R, E), i32, device),
        send_counts=_empty((R, W, R), i32, device), send_offsets=_empty((R, W, R), i32, device),
        recv_counts=_empty((R, W, R), i32, device), recv_offsets=_empty((R, W, R), i32, device),
        expert_counts=_empty((E,), i32, device), expert_offsets=_empty((E,), i32, device),
        pos=_empty((T, k), i32, device),
        workspace=_empty((max(vsrc_workspace_bytes(shape), 1),), torch.uint8, device), rows=rows)


def vsrc_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, shape: Shape, out: dict) -> dict:
    """Every source shard's dispatch into out["send_buf"] plus the count
    exchange tables (four launches)."""
    sh = shape.c()
    _check(lib().moe_vsrc_dispatch(
        ctypes.byref(sh), _ptr(x), _ptr(topk_idx), _ptr(out["send_buf"]), _ptr(out["src_counts"]),
        _ptr(out["src_offsets"]), _ptr(out["send_counts"]), _ptr(out["send_offsets"]), _ptr(out["recv_counts"]),
        _ptr(out["recv_offsets"]), _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["pos"]), _ptr(out["workspace"]), out["workspace"].numel(), _stream()),
        "moe_vsrc_dispatch")
    return out


def vsrc_exchange(src: torch.Tensor, dst: torch.Tensor, shape: Shape, out: dict,
                  direction: int = 0) -> torch.Tensor:
    """The all-to-all as a block transpose: send -> recv (direction 0) or
    recv -> send (direction 1), with the tables in `out`."""
    sh = shape.c()
    _check(lib().moe_vsrc_exchange(
        ctypes.byref(sh), direction, _ptr(src), _ptr(dst), _ptr(out["send_offsets"]),
        _ptr(out["recv_counts"]), _ptr(out["recv_offsets"]), _stream()), "moe_vsrc_exchange")
    return dst


def vsrc_exchange_direct(src: torch.Tensor, dst: torch.Tensor, shape: Shape, out: dict,
                         direction: int = 0) -> torch.Tensor:
    """The exchange straight into the grouped layout: send -> grouped
    (direction 0) or grouped -> send (1), one copy."""
    sh = shape.c()
    _check(lib().moe_vsrc_exchange_direct(
        ctypes.byref(sh), direction, _ptr(src), _ptr(dst), _ptr(out["src_counts"]),
        _ptr(out["src_offsets"]), _ptr(out["expert_offsets"]), _ptr(out["workspace"]),
        out["workspace"].numel(), _stream()), "moe_vsrc_exchange_direct")
    return dst


def vsrc_regroup(src: torch.Tensor, dst: torch.Tensor, shape: Shape, out: dict,
                 direction: int = 0) -> torch.Tensor:
    """Receive-side regroup: recv -> grouped (direction 0) or back (1)."""
    sh = shape.c()
    _check(lib().moe_vsrc_regroup(
        ctypes.byref(sh), direction, _ptr(src), _ptr(dst), _ptr(out["src_counts"]),
        _ptr(out["recv_offsets"]), _ptr(out["expert_offsets"]), _ptr(out["workspace"]),
        out["workspace"].numel(), _stream()), "moe_vsrc_regroup")
    return dst


def expert_scale_rows(send_buf: torch.Tensor, expert_offsets: torch.Tensor,
                      expert_counts: torch.Tensor, shape: Shape,
                      expert_out: torch.Tensor | None = None) -> torch.Tensor:
    expert_out = torch.empty_like(send_buf) if expert_out is None else expert_out
    sh = shape.c()
    _check(lib().moe_expert_scale_rows(ctypes.byref(sh), send_buf.shape[0], _ptr(send_buf),
                                       _ptr(expert_offsets), _ptr(expert_counts),
                                       _ptr(expert_out), _stream()), "moe_expert_scale_rows")
    return expert_out


def combine_rows(expert_out: torch.Tensor, topk_w: torch.Tensor, pos: torch.Tensor, shape: Shape,
                 y: torch.Tensor | None = None) -> torch.Tensor:
    y = _empty((shape.T, shape.H), shape.dtype, expert_out.device) if y is None else y
    sh = shape.c()
    _check(lib().moe_combine_rows(ctypes.byref(sh), expert_out.shape[0], _ptr(expert_out),
                                  _ptr(topk_w), _ptr(pos), _ptr(y), _stream()),
           "moe_combine_rows")
    return y


# ----------------------------------------------------------- expert / combine

def expert_scale(send_buf: torch.Tensor, expert_offsets: torch.Tensor,
                 expert_counts: torch.Tensor, shape: Shape,
                 expert_out: torch.Tensor | None = None) -> torch.Tensor:
    expert_out = torch.empty_like(send_buf) if expert_out is None else expert_out
    sh = shape.c()
    _check(lib().moe_expert_scale(ctypes.byref(sh), _ptr(send_buf), _ptr(expert_offsets),
                                  _ptr(expert_counts), _ptr(expert_out), _stream()),
           "moe_expert_scale")
    return expert_out


def expert_swiglu_workspace_bytes(shape: Shape, I: int) -> int:
    sh = shape.c()
    return int(lib().moe_expert_swiglu_workspace_bytes(ctypes.byref(sh), I))


def expert_swiglu(send_buf: torch.Tensor, expert_offsets: torch.Tensor,
                  expert_counts: torch.Tensor, shape: Shape, w_gate_up: torch.Tensor,
                  w_down: torch.Tensor, expert_out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None,
                  chains: Chains | None = None) -> torch.Tensor:
    """SwiGLU expert FFN on MFMA; w_gate_up [E,2I,H], w_down [E,H,I] bf16. With
    `chains` (a side stream and two events) the odd-id experts run on the side
    stream; without, one chain on the current stream."""
    I = w_down.shape[2]
    expert_out = torch.empty_like(send_buf) if expert_out is None else expert_out
    if workspace is None:
        workspace = _empty((max(expert_swiglu_workspace_bytes(shape, I), 1),), torch.uint8,
                           send_buf.device)
    side, fork, join = None, None, None
    if chains is not None and chains.stream is not None:
        side, fork, join = chains.side_ptr(), chains.event_ptr(0), chains.event_ptr(1)
    sh = shape.c()
    _check(lib().moe_expert_swiglu(ctypes.byref(sh), I, _ptr(send_buf), _ptr(expert_offsets),
                                   _ptr(expert_counts), _ptr(w_gate_up), _ptr(w_down),
                                   _ptr(expert_out), _ptr(workspace), workspace.numel(),
                                   _stream(), side, fork, join), "moe_expert_swiglu")
    return expert_out


def _wave_combine_args(combine: dict | None, shape: Shape, device):
    """(topk_w, pos, token_order, token_wave_offsets, y) pointers of a
    per-wave combine, or five NULLs; the combine stream (NULL: the copy
    stream); y. `combine` holds topk_w, pos, the order tables of
    combine_order(), optionally y (allocated when missing) and optionally
    "stream", a torch stream of the combines' own."""
    if combine is None:
        return (None,) * 5, None, None
    y = combine.get("y")
    if y is None:
        y = _empty((shape.T, shape.H), shape.dtype, device)
    cs = combine.get("stream")
    return ((_ptr(combine["topk_w"]), _ptr(combine["pos"]), _ptr(combine["token_order"]),
             _ptr(combine["token_wave_offsets"]), _ptr(y)),
            None if cs is None else ctypes.c_void_p(cs.cuda_stream), y)


def swiglu_waves(x: torch.Tensor, out: dict, shape: Shape, w_gate_up: torch.Tensor,
                 w_down: torch.Tensor, expert_out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None,
                 copy_stream: torch.cuda.Stream | None = None,
                 chains: Chains | None = None, combine: dict | None = None):
    """Wave-pipelined dispatch + SwiGLU FFN: per wave a gather of its rows into
    out["send_buf"] on `copy_stream`, then the FFN of its experts on the
    current stream after an event. `out` holds a dispatch index of `shape`
    (row_token, wave_offsets, expert offsets/counts). No copy stream: the same
    launches on the current stream. `chains` supplies the events (at least
    swiglu_waves_events(W) of them when a copy stream or a side stream is used)
    and, when it has one, the side stream of the second chain of experts.
    With `combine` (topk_w, pos, token_order, token_wave_offsets, optional y
    and "stream") each wave's completed tokens are combined in the pipeline,
    on that stream or else on the copy stream; returns (expert_out, y) then,
    else expert_out."""
    I = w_down.shape[2]
    send_buf = out["send_buf"]
    expert_out = torch.empty_like(send_buf) if expert_out is None else expert_out
    if workspace is None:
        workspace = _empty((max(expert_swiglu_workspace_bytes(shape, I), 1),), torch.uint8,
                           send_buf.device)
    compute = _stream()
    copy = compute if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
    side = chains.side_ptr() if chains is not None else None
    cargs, cstream, y = _wave_combine_args(combine, shape, send_buf.device)
    if (copy_stream is not None or side is not None or cstream is not None) and (
            chains is None or len(chains.events) < swiglu_waves_events(shape.W)):
        raise ValueError(f"swiglu_waves with a copy, side or combine stream needs a Chains with "
                         f"at least {swiglu_waves_events(shape.W)} events")
    events = chains.event_array() if chains is not None else None
    n_events = len(chains.events) if chains is not None else 0
    sh = shape.c()
    _check(lib().moe_swiglu_waves(
        ctypes.byref(sh), I, _ptr(x), _ptr(out["row_token"]), _ptr(out["wave_offsets"]),
        _ptr(out["expert_offsets"]), _ptr(out["expert_counts"]), _ptr(w_gate_up), _ptr(w_down),
        _ptr(send_buf), _ptr(expert_out), _ptr(workspace), workspace.numel(), *cargs, compute,
        copy, side, cstream, events, n_events), "moe_swiglu_waves")
    return expert_out if combine is None else (expert_out, y)


def scale_waves(x: torch.Tensor, out: dict, shape: Shape, expert_out: torch.Tensor | None = None,
                copy_stream: torch.cuda.Stream | None = None,
                chains: Chains | None = None, combine: dict | None = None):
    """Wave-pipelined dispatch + identity-scaled experts: per wave a gather of its
    rows into out["send_buf"] on `copy_stream`, then the (e+1) scaling of those
    rows on the current stream after an event. `out` holds a dispatch index of
    `shape`; with a copy stream, `chains` supplies at least scale_waves_events(W)
    events. `combine` as in swiglu_waves."""
    send_buf = out["send_buf"]
    expert_out = torch.empty_like(send_buf) if expert_out is None else expert_out
    compute = _stream()
    copy = compute if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
    need = scale_waves_events(shape.W)
    cargs, cstream, y = _wave_combine_args(combine, shape, send_buf.device)
    if (copy_stream is not None or cstream is not None) and (
            chains is None or len(chains.events) < need):
        raise ValueError(f"scale_waves with a copy or combine stream needs a Chains with at "
                         f"least {need} events")
    events = chains.event_array() if chains is not None else None
    n_events = len(chains.events) if chains is not None else 0
    sh = shape.c()
    _check(lib().moe_scale_waves(
        ctypes.byref(sh), _ptr(x), _ptr(out["row_token"]), _ptr(out["wave_offsets"]),
        _ptr(out["expert_offsets"]), _ptr(out["expert_counts"]), _ptr(send_buf),
        _ptr(expert_out), *cargs, compute, copy, cstream, events, n_events), "moe_scale_waves")
    return expert_out if combine is None else (expert_out, y)


def combine_order_workspace_bytes(shape: Shape) -> int:
    sh = shape.c()
    return int(lib().moe_combine_order_workspace_bytes(ctypes.byref(sh)))


def combine_order(pos: torch.Tensor, wave_offsets: torch.Tensor, shape: Shape,
                  token_wave_offsets: torch.Tensor | None = None,
                  token_order: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None):
    """Completion-wave order of the tokens: (token_wave_offsets int32 [W+1],
    token_order int32 [T])."""
    dev = pos.device
    two = _empty((shape.W + 1,), torch.int32, dev) if token_wave_offsets is None \
        else token_wave_offsets
    order = _empty((shape.T,), torch.int32, dev) if token_order is None else token_order
    if workspace is None:
        workspace = _empty((max(combine_order_workspace_bytes(shape), 1),), torch.uint8, dev)
    sh = shape.c()
    _check(lib().moe_combine_order(ctypes.byref(sh), _ptr(pos), _ptr(wave_offsets), _ptr(two),
                                   _ptr(order), _ptr(workspace), workspace.numel(), _stream()),
           "moe_combine_order")
    return two, order


def combine_waves(expert_out: torch.Tensor, topk_w: torch.Tensor, pos: torch.Tensor,
                  token_order: torch.Tensor, token_wave_offsets: torch.Tensor, shape: Shape,
                  w0: int, w1: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """Combine of the tokens whose completion wave lies in [w0, w1) into y."""
    y = _empty((shape.T, shape.H), shape.dtype, expert_out.device) if y is None else y
    sh = shape.c()
    _check(lib().moe_combine_waves(ctypes.byref(sh), _ptr(expert_out), _ptr(topk_w), _ptr(pos),
                                   _ptr(token_order), _ptr(token_wave_offsets), w0, w1, _ptr(y),
                                   _stream()), "moe_combine_waves")
    return y


def combine(expert_out: torch.Tensor, topk_w: torch.Tensor, pos: torch.Tensor, shape: Shape,
            y: torch.Tensor | None = None) -> torch.Tensor:
    y = _empty((shape.T, shape.H), shape.dtype, expert_out.device) if y is None else y
    sh = shape.c()
    _check(lib().moe_combine(ctypes.byref(sh), _ptr(expert_out), _ptr(topk_w), _ptr(pos), _ptr(y),
                             _stream()), "moe_combine")
    return y


# ---------------------------------------------------------------------- stats

def stats_device(expert_counts: torch.Tensor, R: int, out: torch.Tensor | None = None):
    """Enqueue the statistics kernel; returns the raw device struct (uint8 tensor)."""
    E = expert_counts.numel()
    out = _empty((STATS_BYTES,), torch.uint8, expert_counts.device) if out is None else out
    _check(lib().moe_stats(_ptr(expert_counts), E, R, _ptr(out), _stream()), "moe_stats")
    return out


def stats_to_dict(raw: torch.Tensor) -> dict:
    s = MoeStats.from_buffer_copy(raw.cpu().numpy().tobytes())
    return {name: getattr(s, name) for name, _ in MoeStats._fields_}


def stats(expert_counts: torch.Tensor, R: int) -> dict:
    """Statistics as a host dict (synchronises with the stream)."""
    return stats_to_dict(stats_device(expert_counts, R))


def dirichlet_alpha_device(expert_counts: torch.Tensor, out: torch.Tensor | None = None):
    """Enqueue the alpha fit; returns the device float64 tensor (one element)."""
    out = _empty((1,), torch.float64, expert_counts.device) if out is None else out
    _check(lib().moe_dirichlet_alpha(_ptr(expert_counts), expert_counts.numel(), _ptr(out),
                                     _stream()), "moe_dirichlet_alpha")
    return out


def dirichlet_alpha(expert_counts: torch.Tensor) -> float:
    """Fitted symmetric Dirichlet alpha of the counts (synchronises)."""
    return float(dirichlet_alpha_device(expert_counts).item())

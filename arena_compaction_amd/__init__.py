"""Python binding for libarena_compaction.so (gfx950).

Argument marshalling only: every step of the compaction runs in the HIP
kernels behind the C-ABI declared in include/arena_compaction.h.  PyTorch is
used for device memory and streams.  Importing this module fails loudly if
the library has not been built -- there is no CPU fallback.

Tables are torch tensors on the GPU: offset and size as int64 holding the
unsigned 64-bit values, live as uint8 (or None: every entry live), pinned as
uint8 (or None: nothing pinned).  Handles
and new offsets are int64 tensors holding unsigned values; an unmapped handle
reads back as -1 (UINT64_MAX).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libarena_compaction.so")

DEFRAG_OK = 0
DEFRAG_EINVAL = -1
DEFRAG_EWORKSPACE = -2
DEFRAG_ENOPLAN = -3
DEFRAG_EHIP = -4
DEFRAG_ETIMEOUT = -5
DEFRAG_ENOFIT = -6
DEFRAG_ECAPACITY = -7
DEFRAG_ECORRUPT = -8
DEFRAG_ETOOBIG = -9
STATIC_SCRATCH_BYTES = 128 << 20   # DEFRAG_STATIC_SCRATCH_BYTES
REASONS = {0: "none", 1: "zero_size", 2: "misaligned", 3: "live_flag",
           4: "out_of_arena", 5: "overlap", 6: "argument", 7: "pinned_flag"}
U64_MAX = (1 << 64) - 1


class defrag_table(ctypes.Structure):
    _fields_ = [("offset_dev", ctypes.c_void_p), ("size_dev", ctypes.c_void_p),
                ("live_dev", ctypes.c_void_p), ("n", ctypes.c_uint64),
                ("pinned_dev", ctypes.c_void_p)]


class defrag_stats_t(ctypes.Structure):
    _fields_ = [(k, ctypes.c_uint64) for k in (
        "arena_bytes", "live_bytes", "free_bytes", "largest_hole", "hole_count",
        "live_blocks", "moved_blocks", "moved_bytes")] + [
        ("frag_free_over_largest_minus_1", ctypes.c_double),
        ("frag_one_minus_largest_over_free", ctypes.c_double),
        ("invalid_index", ctypes.c_uint64), ("invalid_reason", ctypes.c_int32),
        ("reserved", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class defrag_tuning(ctypes.Structure):
    _fields_ = [("tile_bytes", ctypes.c_uint32), ("wg_per_cu", ctypes.c_uint32),
                ("nontemporal", ctypes.c_uint32), ("spin_limit_log2", ctypes.c_uint32),
                ("stall_every", ctypes.c_uint32), ("stall_sleeps", ctypes.c_uint32),
                ("stall_seed", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class defrag_move_report_t(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("tiles", ctypes.c_uint64), ("late_tiles", ctypes.c_uint64),
                ("waited_tiles", ctypes.c_uint64), ("polls", ctypes.c_uint64)]


class defrag_plan_t(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint64), ("epoch", ctypes.c_uint64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
                ("n", ctypes.c_uint64), ("arena_bytes", ctypes.c_uint64),
                ("live_blocks", ctypes.c_uint64), ("pinned_blocks", ctypes.c_uint64),
                ("move_begin", ctypes.c_uint64), ("live_bytes", ctypes.c_uint64),
                ("n_tiles", ctypes.c_uint64), ("max_tiles", ctypes.c_uint64),
                ("max_blocks_per_tile", ctypes.c_uint64), ("whole_tiles", ctypes.c_uint64),
                ("request_bytes", ctypes.c_uint64), ("window_begin", ctypes.c_uint64),
                ("window_end", ctypes.c_uint64), ("window_hole", ctypes.c_uint64),
                ("state", ctypes.c_int32), ("device", ctypes.c_int32),
                ("tuning", defrag_tuning), ("stats", defrag_stats_t)]


class defrag_monitor_cfg(ctypes.Structure):
    _fields_ = [("warning_ratio", ctypes.c_double), ("critical_ratio", ctypes.c_double),
                ("frag_threshold", ctypes.c_double), ("next_request", ctypes.c_uint64),
                ("growth_bytes_per_s", ctypes.c_double)]


class defrag_monitor_report(ctypes.Structure):
    _fields_ = [("level", ctypes.c_int32), ("action", ctypes.c_int32),
                ("usage_ratio", ctypes.c_double),
                ("frag_free_over_largest_minus_1", ctypes.c_double),
                ("frag_one_minus_largest_over_free", ctypes.c_double),
                ("seconds_to_full", ctypes.c_double)]


LEVELS = {0: "OK", 1: "WARNING", 2: "CRITICAL"}
ACTIONS = {0: "none", 1: "targeted", 2: "full", 3: "no_room"}


class defrag_compact_args(ctypes.Structure):
    _fields_ = [("table", ctypes.POINTER(defrag_table)), ("arena_bytes", ctypes.c_uint64),
                ("arena_dev", ctypes.c_void_p), ("request_bytes", ctypes.c_uint64),
                ("tuning", ctypes.POINTER(defrag_tuning)), ("ws_dev", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t), ("new_offset_dev", ctypes.c_void_p),
                ("h_in_dev", ctypes.c_void_p), ("h_out_dev", ctypes.c_void_p),
                ("n_handles", ctypes.c_uint64), ("n_invalid_dev", ctypes.c_void_p),
                ("offset_out_dev", ctypes.c_void_p), ("size_out_dev", ctypes.c_void_p),
                ("live_out_dev", ctypes.c_void_p), ("pinned_out_dev", ctypes.c_void_p)]


# defrag_tile_t: one mover tile of a plan (defrag_plan_tiles)
TILE_DTYPE = np.dtype([("dst_begin", "<u8"), ("dst_end", "<u8"), ("shift_first", "<u8"),
                       ("first_block", "<u4"), ("last_block", "<u4"),
                       ("dep_lo", "<u4"), ("dep_hi", "<u4")])
assert TILE_DTYPE.itemsize == 40


class DefragError(RuntimeError):
    def __init__(self, code: int, what: str, stats: Optional[defrag_stats_t] = None):
        self.code = code
        self.invalid_index = None
        self.invalid_reason = None
        msg = f"{what}: {strerror(code)} ({code})"
        if stats is not None and stats.invalid_reason:
            self.invalid_index = int(stats.invalid_index)
            self.invalid_reason = int(stats.invalid_reason)
            msg += f"; entry {self.invalid_index}: {REASONS.get(self.invalid_reason, '?')}"
        super().__init__(msg)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
            "g.build()'); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, U, S = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_size_t
    L.defrag_workspace_bytes.argtypes = [U, U, U, ctypes.c_uint32]
    L.defrag_workspace_bytes.restype = S
    L.defrag_stats.argtypes = [ctypes.POINTER(defrag_table), U, P, S, P,
                               ctypes.POINTER(defrag_stats_t)]
    L.defrag_plan.argtypes = [ctypes.POINTER(defrag_table), U, ctypes.POINTER(defrag_tuning),
                              P, S, P, P, ctypes.POINTER(defrag_plan_t)]
    L.defrag_plan_targeted.argtypes = [ctypes.POINTER(defrag_table), U, U,
                                       ctypes.POINTER(defrag_tuning), P, S, P, P,
                                       ctypes.POINTER(defrag_plan_t)]
    L.defrag_first_fit.argtypes = [ctypes.POINTER(defrag_table), U, U, P, S, P,
                                   ctypes.POINTER(ctypes.c_uint64),
                                   ctypes.POINTER(defrag_stats_t)]
    L.defrag_move.argtypes = [P, U, ctypes.POINTER(defrag_plan_t), P, S, P]
    L.defrag_move_status.argtypes = [ctypes.POINTER(defrag_plan_t), P, P]
    L.defrag_move_report.argtypes = [ctypes.POINTER(defrag_plan_t), P, P,
                                     ctypes.POINTER(defrag_move_report_t)]
    L.defrag_plan_tiles.argtypes = [ctypes.POINTER(defrag_plan_t), P, S, P, U, P]
    L.defrag_remap.argtypes = [ctypes.POINTER(defrag_plan_t), P, S, P, P, U, P, P]
    L.defrag_commit.argtypes = [ctypes.POINTER(defrag_plan_t), P, S, P, P, P, P, P]
    L.defrag_compact.argtypes = [ctypes.POINTER(defrag_compact_args), P,
                                 ctypes.POINTER(defrag_plan_t), ctypes.POINTER(defrag_stats_t)]
    L.defrag_compact_static.argtypes = [ctypes.POINTER(defrag_compact_args), P,
                                        ctypes.POINTER(defrag_plan_t),
                                        ctypes.POINTER(defrag_stats_t)]
    L.defrag_monitor.argtypes = [ctypes.POINTER(defrag_stats_t), ctypes.POINTER(defrag_monitor_cfg),
                                 ctypes.POINTER(defrag_monitor_report)]
    L.defrag_strerror.argtypes = [ctypes.c_int]
    L.defrag_strerror.restype = ctypes.c_char_p
    for f in ("defrag_stats", "defrag_first_fit", "defrag_plan", "defrag_plan_targeted",
              "defrag_move", "defrag_monitor", "defrag_compact", "defrag_compact_static",
              "defrag_move_status", "defrag_move_report", "defrag_plan_tiles",
              "defrag_remap", "defrag_commit"):
        getattr(L, f).restype = ctypes.c_int
    return L


lib = _load()

EXPORTS = ("defrag_workspace_bytes", "defrag_stats", "defrag_first_fit", "defrag_plan",
           "defrag_plan_targeted",
           "defrag_move",
           "defrag_move_status", "defrag_move_report", "defrag_plan_tiles", "defrag_remap",
           "defrag_commit",
           "defrag_compact", "defrag_compact_static", "defrag_monitor",
           "defrag_strerror")


def strerror(code: int) -> str:
    return lib.defrag_strerror(int(code)).decode()


def _ptr(t: Optional[torch.Tensor]):
    """The device address of t (an int: every pointer argument and field is
    declared c_void_p, which takes one as it is)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError("device arguments must be contiguous GPU tensors")
    return t.data_ptr()


def _need(t: Optional[torch.Tensor], dtype: torch.dtype, n: int, what: str) -> None:
    """Raise unless t is None or a tensor of dtype with at least n elements
    (the kernels write or read that many; a shorter buffer would be overrun)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise ValueError(f"{what}: expected a {dtype} tensor")
    if t.numel() < n:
        raise ValueError(f"{what}: {t.numel()} elements, {n} needed")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_table(offset: torch.Tensor, size: torch.Tensor, live: Optional[torch.Tensor],
               pinned: Optional[torch.Tensor] = None) -> defrag_table:
    n = offset.numel()
    _need(offset, torch.int64, 0, "offset")
    _need(size, torch.int64, n, "size")
    _need(live, torch.uint8, n, "live")
    _need(pinned, torch.uint8, n, "pinned")
    return defrag_table(_ptr(offset) if n else None, _ptr(size) if n else None,
                        _ptr(live) if (live is not None and n) else None, n,
                        _ptr(pinned) if (pinned is not None and n) else None)


def defrag_workspace_bytes(n: int, arena_bytes: int, tile_bytes: int = 0,
                           max_pinned: int = 0) -> int:
    return int(lib.defrag_workspace_bytes(n, max_pinned, arena_bytes, tile_bytes))


def workspace(n: int, arena_bytes: int, tile_bytes: int = 0, device=None,
              max_pinned: int = 0) -> torch.Tensor:
    """Allocate a workspace tensor (torch allocations are 256-byte aligned)."""
    nb = defrag_workspace_bytes(n, arena_bytes, tile_bytes, max_pinned)
    if nb == 0:
        raise DefragError(DEFRAG_EINVAL, "defrag_workspace_bytes")
    return torch.empty(nb, dtype=torch.uint8, device=device or "cuda")


def defrag_stats(offset, size, live, arena_bytes: int, ws: torch.Tensor,
                 stream=None, pinned=None) -> defrag_stats_t:
    t = make_table(offset, size, live, pinned)
    out = defrag_stats_t()
    rc = lib.defrag_stats(ctypes.byref(t), arena_bytes, _ptr(ws), ws.numel(), _stream(stream),
                          ctypes.byref(out))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_stats", out)
    return out


def defrag_first_fit(offset, size, live, arena_bytes: int, request_bytes: int,
                     ws: torch.Tensor, stream=None, pinned=None):
    """(offset, stats): the offset first fit gives the request, or None when
    no hole holds it (DEFRAG_ENOFIT)."""
    t = make_table(offset, size, live, pinned)
    out = ctypes.c_uint64()
    st = defrag_stats_t()
    rc = lib.defrag_first_fit(ctypes.byref(t), arena_bytes, request_bytes, _ptr(ws), ws.numel(),
                              _stream(stream), ctypes.byref(out), ctypes.byref(st))
    if rc == DEFRAG_ENOFIT:
        return None, st
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_first_fit", st)
    return int(out.value), st


def defrag_plan(offset, size, live, arena_bytes: int, ws: torch.Tensor,
                new_offset: Optional[torch.Tensor] = None,
                tuning: Optional[defrag_tuning] = None, stream=None,
                pinned: Optional[torch.Tensor] = None) -> defrag_plan_t:
    _need(new_offset, torch.int64, offset.numel(), "new_offset")
    t = make_table(offset, size, live, pinned)
    plan = defrag_plan_t()
    rc = lib.defrag_plan(ctypes.byref(t), arena_bytes,
                         ctypes.byref(tuning) if tuning is not None else None,
                         _ptr(ws), ws.numel(), _stream(stream),
                         _ptr(new_offset) if new_offset is not None and new_offset.numel() else None,
                         ctypes.byref(plan))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_plan", plan.stats)
    return plan


def defrag_plan_targeted(offset, size, live, arena_bytes: int, request_bytes: int,
                         ws: torch.Tensor, new_offset: Optional[torch.Tensor] = None,
                         tuning: Optional[defrag_tuning] = None, stream=None,
                         pinned: Optional[torch.Tensor] = None) -> defrag_plan_t:
    """Raises DefragError with code DEFRAG_ENOFIT when no window fits."""
    _need(new_offset, torch.int64, offset.numel(), "new_offset")
    t = make_table(offset, size, live, pinned)
    plan = defrag_plan_t()
    rc = lib.defrag_plan_targeted(ctypes.byref(t), arena_bytes, request_bytes,
                                  ctypes.byref(tuning) if tuning is not None else None,
                                  _ptr(ws), ws.numel(), _stream(stream),
                                  _ptr(new_offset) if new_offset is not None and new_offset.numel()
                                  else None, ctypes.byref(plan))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_plan_targeted", plan.stats)
    return plan


def defrag_move(arena: torch.Tensor, plan: defrag_plan_t, ws: torch.Tensor, stream=None) -> None:
    _need(arena, torch.uint8, 0, "arena")
    rc = lib.defrag_move(_ptr(arena) if arena.numel() else None, arena.numel(),
                         ctypes.byref(plan), _ptr(ws), ws.numel(), _stream(stream))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_move")


def defrag_move_status(plan: defrag_plan_t, ws: torch.Tensor, stream=None) -> int:
    return int(lib.defrag_move_status(ctypes.byref(plan), _ptr(ws), _stream(stream)))


def defrag_move_report(plan: defrag_plan_t, ws: torch.Tensor, stream=None) -> defrag_move_report_t:
    """The move's outcome (status) and the mover's wait counters."""
    out = defrag_move_report_t()
    rc = lib.defrag_move_report(ctypes.byref(plan), _ptr(ws), _stream(stream), ctypes.byref(out))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_move_report")
    return out


def defrag_plan_tiles(plan: defrag_plan_t, ws: torch.Tensor, stream=None) -> np.ndarray:
    """The plan's mover tiles as a structured array of TILE_DTYPE."""
    n = int(plan.n_tiles)
    out = np.zeros(n, dtype=TILE_DTYPE)
    rc = lib.defrag_plan_tiles(ctypes.byref(plan), _ptr(ws), ws.numel(),
                               ctypes.c_void_p(out.ctypes.data) if n else None, n,
                               _stream(stream))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_plan_tiles")
    return out


def defrag_remap(plan: defrag_plan_t, ws: torch.Tensor, h_in: torch.Tensor,
                 h_out: Optional[torch.Tensor] = None,
                 n_invalid: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _need(h_in, torch.int64, 0, "h_in")
    if h_out is None:
        h_out = torch.empty_like(h_in)
    H = h_in.numel()
    _need(h_out, torch.int64, H, "h_out")
    _need(n_invalid, torch.int64, 1, "n_invalid")
    rc = lib.defrag_remap(ctypes.byref(plan), _ptr(ws), ws.numel(),
                          _ptr(h_in) if H else None, _ptr(h_out) if H else None, H,
                          _ptr(n_invalid), _stream(stream))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_remap")
    return h_out


def defrag_commit(plan: defrag_plan_t, ws: torch.Tensor, offset_out=None, size_out=None,
                  live_out=None, stream=None, pinned_out=None) -> None:
    m = int(plan.live_blocks)
    _need(offset_out, torch.int64, m, "offset_out")
    _need(size_out, torch.int64, m, "size_out")
    _need(live_out, torch.uint8, m, "live_out")
    _need(pinned_out, torch.uint8, m, "pinned_out")
    rc = lib.defrag_commit(ctypes.byref(plan), _ptr(ws), ws.numel(), _ptr(offset_out),
                           _ptr(size_out), _ptr(live_out), _ptr(pinned_out), _stream(stream))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_commit")


def _compact_args(offset, size, live, arena_bytes, arena, ws, request_bytes, new_offset, handles,
                  h_out, n_invalid, offset_out, size_out, live_out, pinned_out, tuning, pinned):
    """The defrag_compact_args of a call, its argument checks, and the
    buffers it points at (kept alive with it)."""
    _need(arena, torch.uint8, 0, "arena")
    _need(new_offset, torch.int64, offset.numel(), "new_offset")
    H = 0 if handles is None else handles.numel()
    if handles is not None:
        _need(handles, torch.int64, 0, "handles")
        if h_out is None:
            h_out = torch.empty_like(handles)
        _need(h_out, torch.int64, H, "h_out")
    _need(n_invalid, torch.int64, 1, "n_invalid")
    for o, dt, name in ((offset_out, torch.int64, "offset_out"), (size_out, torch.int64, "size_out"),
                        (live_out, torch.uint8, "live_out"), (pinned_out, torch.uint8, "pinned_out")):
        _need(o, dt, 0, name)
    t = make_table(offset, size, live, pinned)
    a = defrag_compact_args(
        ctypes.pointer(t), arena_bytes, _ptr(arena) if arena.numel() else None, request_bytes,
        ctypes.pointer(tuning) if tuning is not None else None,
        _ptr(ws) if ws is not None else None, ws.numel() if ws is not None else 0,
        _ptr(new_offset) if new_offset is not None and new_offset.numel() else None,
        _ptr(handles) if H else None, _ptr(h_out) if H else None, H, _ptr(n_invalid),
        _ptr(offset_out) if offset_out is not None and offset_out.numel() else None,
        _ptr(size_out) if size_out is not None and size_out.numel() else None,
        _ptr(live_out) if live_out is not None and live_out.numel() else None,
        _ptr(pinned_out) if pinned_out is not None and pinned_out.numel() else None)
    return a, (t, h_out)


def defrag_compact(offset, size, live, arena_bytes: int, arena: torch.Tensor, ws: torch.Tensor,
                   request_bytes: int = 0, new_offset: Optional[torch.Tensor] = None,
                   handles: Optional[torch.Tensor] = None, h_out: Optional[torch.Tensor] = None,
                   n_invalid: Optional[torch.Tensor] = None, offset_out=None, size_out=None,
                   live_out=None, pinned_out=None, tuning: Optional[defrag_tuning] = None,
                   stream=None, pinned=None, after: Optional[bool] = None):
    """Plan, move, remap, commit and the post-check in one C-ABI call.
    after (default: whenever offset_out and size_out are given) asks for the
    post-move statistics.  Returns (plan, post-move stats or None).
    offset_out, size_out, live_out and pinned_out need one element per live
    block, which is known only once the plan has run: neither this function
    nor the library can check their length."""
    if after is None:
        after = offset_out is not None and size_out is not None
    a, keep = _compact_args(offset, size, live, arena_bytes, arena, ws, request_bytes, new_offset,
                            handles, h_out, n_invalid, offset_out, size_out, live_out, pinned_out,
                            tuning, pinned)
    plan = defrag_plan_t()
    post = defrag_stats_t() if after else None
    rc = lib.defrag_compact(ctypes.byref(a), _stream(stream), ctypes.byref(plan),
                            ctypes.byref(post) if after else None)
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_compact", plan.stats if rc == DEFRAG_EINVAL else None)
    return plan, post


def defrag_compact_static(offset, size, live, arena_bytes: int, arena: torch.Tensor,
                          request_bytes: int = 0, new_offset: Optional[torch.Tensor] = None,
                          handles: Optional[torch.Tensor] = None,
                          h_out: Optional[torch.Tensor] = None,
                          n_invalid: Optional[torch.Tensor] = None, offset_out=None,
                          size_out=None, live_out=None, pinned_out=None,
                          tuning: Optional[defrag_tuning] = None, stream=None, pinned=None,
                          after: Optional[bool] = None):
    """defrag_compact with the library's static scratch as its workspace:
    the library allocates nothing and creates no stream or event for it
    (every step runs on `stream`).  Returns (plan, post-move stats or None);
    DEFRAG_ETOOBIG when the table needs more than the scratch holds."""
    if after is None:
        after = offset_out is not None and size_out is not None
    a, keep = _compact_args(offset, size, live, arena_bytes, arena, None, request_bytes,
                            new_offset, handles, h_out, n_invalid, offset_out, size_out, live_out,
                            pinned_out, tuning, pinned)
    plan = defrag_plan_t()
    post = defrag_stats_t() if after else None
    rc = lib.defrag_compact_static(ctypes.byref(a), _stream(stream), ctypes.byref(plan),
                                   ctypes.byref(post) if after else None)
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_compact_static",
                          plan.stats if rc == DEFRAG_EINVAL else None)
    return plan, post


def defrag_monitor(stats: defrag_stats_t, warning_ratio: float = 0.85,
                   critical_ratio: float = 0.95, frag_threshold: float = 0.0,
                   next_request: int = 0, growth_bytes_per_s: float = 0.0) -> defrag_monitor_report:
    cfg = defrag_monitor_cfg(warning_ratio, critical_ratio, frag_threshold, next_request,
                             growth_bytes_per_s)
    out = defrag_monitor_report()
    rc = lib.defrag_monitor(ctypes.byref(stats), ctypes.byref(cfg), ctypes.byref(out))
    if rc != DEFRAG_OK:
        raise DefragError(rc, "defrag_monitor")
    return out


def defrag_strerror(code: int) -> str:
    return strerror(code)

"""ctypes loader for the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP library.
"""
from __future__ import annotations

import collections
import ctypes
import dataclasses
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "oracle.cpp")]

OK = 0
EINVAL = -1
REASONS = {0: "none", 1: "zero_size", 2: "misaligned", 3: "live_flag",
           4: "out_of_arena", 5: "overlap", 7: "pinned_flag"}
U64_MAX = (1 << 64) - 1


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with g++ (plain -O2, single-threaded)."""
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall", "-Wextra",
           "-o", LIB_PATH + ".tmp"] + SOURCES
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Stats(ctypes.Structure):
    _fields_ = [(k, ctypes.c_uint64) for k in (
        "arena_bytes", "live_bytes", "free_bytes", "largest_hole", "hole_count",
        "live_blocks", "moved_blocks", "moved_bytes")] + [
        ("frag_free_over_largest_minus_1", ctypes.c_double),
        ("frag_one_minus_largest_over_free", ctypes.c_double)]


@dataclasses.dataclass(frozen=True)
class Stats:
    arena_bytes: int
    live_bytes: int
    free_bytes: int
    largest_hole: int
    hole_count: int
    live_blocks: int
    moved_blocks: int
    moved_bytes: int
    frag_free_over_largest_minus_1: float
    frag_one_minus_largest_over_free: float


_lib = None


def _bind(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    U = ctypes.c_uint64
    L.oracle_validate.argtypes = [P, P, P, P, U, U, P, P]
    L.oracle_validate.restype = ctypes.c_int
    L.oracle_new_offsets.argtypes = [P, P, P, P, U, P]
    L.oracle_compact.argtypes = [P, U, P, P, P, P, U]
    L.oracle_stats_walk.argtypes = [P, P, P, P, U, U, P]
    L.oracle_remap.argtypes = [P, P, P, P, U, P, P, U, P]
    L.oracle_source_map.argtypes = [P, P, P, P, U, U, U, U, P, P, P, U]
    L.oracle_source_map.restype = ctypes.c_int64
    L.oracle_target_window.argtypes = [P, P, P, P, U, U, U, P]
    L.oracle_target_window.restype = ctypes.c_int
    L.oracle_first_fit.argtypes = [P, P, P, U, U, U, P]
    L.oracle_first_fit.restype = ctypes.c_int
    D = ctypes.c_double
    L.oracle_monitor.argtypes = [U, U, U, D, D, D, U, D, P]
    return L


def swap_library(path: str):
    """Load the oracle from another build (tests use it to check that the
    pins reject deliberately broken copies).  Returns the previous handle;
    pass it to restore_library."""
    global _lib
    prev = lib()
    _lib = _bind(path)
    return prev


def restore_library(handle) -> None:
    global _lib
    _lib = handle


def lib():
    global _lib
    if _lib is None:
        stale = (not os.path.exists(LIB_PATH) or
                 any(os.path.getmtime(f) > os.path.getmtime(LIB_PATH)
                     for f in SOURCES + [os.path.join(HERE, "oracle.h")]))
        if stale:
            build()
        _lib = _bind(LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _table(off, size, live, pinned=None):
    off = np.ascontiguousarray(off, dtype=np.uint64)
    size = np.ascontiguousarray(size, dtype=np.uint64)
    live = np.ascontiguousarray(live, dtype=np.uint8)
    assert off.shape == size.shape == live.shape
    if pinned is not None:
        pinned = np.ascontiguousarray(pinned, dtype=np.uint8)
        assert pinned.shape == off.shape
    return off, size, live, pinned


def validate(off, size, live, arena_bytes, pinned=None):
    off, size, live, pinned = _table(off, size, live, pinned)
    bad = ctypes.c_uint64()
    reason = ctypes.c_int32()
    rc = lib().oracle_validate(_p(off), _p(size), _p(live), _p(pinned), off.shape[0],
                               arena_bytes, ctypes.byref(bad), ctypes.byref(reason))
    return rc, bad.value, reason.value


def new_offsets(off, size, live, pinned=None):
    off, size, live, pinned = _table(off, size, live, pinned)
    out = np.empty(off.shape[0], dtype=np.uint64)
    lib().oracle_new_offsets(_p(off), _p(size), _p(live), _p(pinned), off.shape[0], _p(out))
    return out


def compact(arena: np.ndarray, off, size, live, pinned=None):
    """In place on a host uint8 arena."""
    assert arena.dtype == np.uint8 and arena.flags["C_CONTIGUOUS"]
    off, size, live, pinned = _table(off, size, live, pinned)
    lib().oracle_compact(_p(arena), arena.shape[0], _p(off), _p(size), _p(live), _p(pinned),
                         off.shape[0])


def stats(off, size, live, arena_bytes, pinned=None) -> Stats:
    off, size, live, pinned = _table(off, size, live, pinned)
    s = _Stats()
    lib().oracle_stats_walk(_p(off), _p(size), _p(live), _p(pinned), off.shape[0],
                            arena_bytes, ctypes.byref(s))
    return Stats(*[getattr(s, f[0]) for f in _Stats._fields_])


def remap(off, size, live, handles, pinned=None):
    off, size, live, pinned = _table(off, size, live, pinned)
    h = np.ascontiguousarray(handles, dtype=np.uint64)
    out = np.empty_like(h)
    bad = ctypes.c_uint64()
    lib().oracle_remap(_p(off), _p(size), _p(live), _p(pinned), off.shape[0], _p(h), _p(out),
                       h.shape[0], ctypes.byref(bad))
    return out, bad.value


def source_map(off, size, live, arena_bytes, p0, length, cap=1 << 16, pinned=None):
    off, size, live, pinned = _table(off, size, live, pinned)
    d = np.empty(cap, dtype=np.uint64)
    s = np.empty(cap, dtype=np.uint64)
    l = np.empty(cap, dtype=np.uint64)
    k = lib().oracle_source_map(_p(off), _p(size), _p(live), _p(pinned), off.shape[0],
                                arena_bytes, p0, length, _p(d), _p(s), _p(l), cap)
    if k < 0:
        raise ValueError("source map needs more pieces than cap")
    return d[:k].copy(), s[:k].copy(), l[:k].copy()


class _Window(ctypes.Structure):
    _fields_ = [(k, ctypes.c_uint64) for k in ("found", "begin", "end", "hole", "moved_bytes")]


Window = collections.namedtuple("Window", [f[0] for f in _Window._fields_])


def target_window(off, size, live, arena_bytes, request, pinned=None) -> Window:
    """The window targeted compaction packs (oracle.h); raises ValueError for
    request == 0."""
    off, size, live, pinned = _table(off, size, live, pinned)
    w = _Window()
    rc = lib().oracle_target_window(_p(off), _p(size), _p(live), _p(pinned), off.shape[0],
                                    arena_bytes, request, ctypes.byref(w))
    if rc != 0:
        raise ValueError("request must be at least one byte")
    return Window(*[getattr(w, f[0]) for f in _Window._fields_])


def window_pins(off, live, pinned, window: Window) -> np.ndarray:
    """Targeted compaction is segmented compaction in which every live block
    outside the window is held in place: the pinned flags that say so."""
    off = np.asarray(off, dtype=np.uint64)
    live = np.asarray(live, dtype=np.uint8)
    outside = (off < np.uint64(window.begin)) | (off >= np.uint64(window.end))
    fixed = (live == 1) & outside
    if pinned is not None:
        fixed |= np.asarray(pinned, dtype=np.uint8) == 1
    return fixed.astype(np.uint8)


def first_fit(off, size, live, arena_bytes, request) -> int:
    """Offset the CANN pool's first fit gives the request (oracle.h), or
    U64_MAX when no hole holds it; ValueError for request == 0."""
    off, size, live, _ = _table(off, size, live)
    out = ctypes.c_uint64()
    rc = lib().oracle_first_fit(_p(off), _p(size), _p(live), off.shape[0], arena_bytes, request,
                                ctypes.byref(out))
    if rc != 0:
        raise ValueError("request must be at least one byte")
    return out.value


class _MonitorOut(ctypes.Structure):
    _fields_ = [("level", ctypes.c_int32), ("action", ctypes.c_int32),
                ("usage_ratio", ctypes.c_double),
                ("frag_free_over_largest_minus_1", ctypes.c_double),
                ("seconds_to_full", ctypes.c_double)]


Monitor = collections.namedtuple("Monitor", [f[0] for f in _MonitorOut._fields_])
LEVELS = {0: "OK", 1: "WARNING", 2: "CRITICAL"}
ACTIONS = {0: "none", 1: "targeted", 2: "full", 3: "no_room"}


def monitor(arena_bytes, live_bytes, largest_hole, warning_ratio=0.85, critical_ratio=0.95,
            frag_threshold=0.0, next_request=0, growth_bytes_per_s=0.0) -> Monitor:
    o = _MonitorOut()
    lib().oracle_monitor(arena_bytes, live_bytes, largest_hole, warning_ratio, critical_ratio,
                         frag_threshold, next_request, growth_bytes_per_s, ctypes.byref(o))
    return Monitor(*[getattr(o, f[0]) for f in _MonitorOut._fields_])

"""Shared test plumbing: run a heap through the HIP path (C-ABI) and through
the oracle, and compare.  Inputs come from workloads only; expected values
come from the oracle only."""
from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import torch

import oracle
import workloads as W

U64_MAX = (1 << 64) - 1
STAT_KEYS = ("arena_bytes", "live_bytes", "free_bytes", "largest_hole", "hole_count",
             "live_blocks", "moved_blocks", "moved_bytes",
             "frag_free_over_largest_minus_1", "frag_one_minus_largest_over_free")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def u64_to_t(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint64).view(np.int64)).to(dev)


def t_to_u64(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


@dataclasses.dataclass
class GpuRun:
    plan: object
    new_off: np.ndarray
    remapped: np.ndarray
    n_invalid: int
    post_stats: object
    status: int
    arena: Optional[torch.Tensor]   # device arena after the move (kept on device)
    ws: torch.Tensor


def device_table(heap: W.Heap, dev):
    return (u64_to_t(heap.offset, dev), u64_to_t(heap.size, dev),
            torch.from_numpy(heap.live).to(dev))


def device_pinned(heap: W.Heap, dev):
    return None if heap.pinned is None else torch.from_numpy(heap.pinned).to(dev)


def pristine_host(heap: W.Heap) -> torch.Tensor:
    t = torch.empty(heap.arena_bytes, dtype=torch.uint8)
    W.fill_payload(t, 0, heap.payload_mode, heap.payload_seed)
    return t


def run_gpu(heap: W.Heap, dev="cuda", tuning=None, arena: Optional[torch.Tensor] = None,
            handles: Optional[np.ndarray] = None, request: Optional[int] = None) -> GpuRun:
    """Plan (targeted when request is given), move, remap, commit and the
    post-move statistics through the C-ABI."""
    import arena_compaction_amd as ac
    off, size, live = device_table(heap, dev)
    pin = device_pinned(heap, dev)
    ws = ac.workspace(heap.n, heap.arena_bytes,
                      tuning.tile_bytes if tuning is not None else 0, device=dev,
                      max_pinned=heap.n_pinned)
    new_off = torch.full((heap.n,), -7, dtype=torch.int64, device=dev)
    if request is None:
        plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws, new_off, tuning=tuning,
                              pinned=pin)
    else:
        plan = ac.defrag_plan_targeted(off, size, live, heap.arena_bytes, request, ws, new_off,
                                       tuning=tuning, pinned=pin)
    if arena is None:
        arena = torch.empty(heap.arena_bytes, dtype=torch.uint8, device=dev)
        W.fill_payload(arena, 0, heap.payload_mode, heap.payload_seed)
    ac.defrag_move(arena, plan, ws)
    status = ac.defrag_move_status(plan, ws)
    hs = heap.handles if handles is None else handles
    h = u64_to_t(hs, dev)
    n_bad = torch.full((1,), -3, dtype=torch.int64, device=dev)
    h_out = ac.defrag_remap(plan, ws, h, n_invalid=n_bad)
    m = int(plan.live_blocks)
    c_off = torch.empty(m, dtype=torch.int64, device=dev)
    c_size = torch.empty(m, dtype=torch.int64, device=dev)
    c_live = torch.zeros(m, dtype=torch.uint8, device=dev)
    c_pin = torch.full((m,), 9, dtype=torch.uint8, device=dev)
    ac.defrag_commit(plan, ws, c_off, c_size, c_live, pinned_out=c_pin)
    post = ac.defrag_stats(c_off, c_size, c_live, heap.arena_bytes, ws, pinned=c_pin)
    torch.cuda.synchronize()
    assert bool((c_live == 1).all()), "commit must mark every packed entry live"
    want_pin = (np.zeros(m, np.uint8) if heap.pinned is None
                else heap.pinned[np.flatnonzero(heap.live)])
    assert np.array_equal(c_pin.cpu().numpy(), want_pin), "commit's pinned flags differ"
    return GpuRun(plan, t_to_u64(new_off), t_to_u64(h_out), int(n_bad.item()), post, status,
                  arena, ws)


def run_gpu_compact(heap: W.Heap, arena: torch.Tensor, request: int = 0,
                    tuning=None) -> GpuRun:
    """The whole operator through one C-ABI call (defrag_compact): plan
    (targeted when request > 0), move, remap, commit and post-check."""
    import arena_compaction_amd as ac
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes, tuning.tile_bytes if tuning else 0,
                      max_pinned=heap.n_pinned)
    new_off = torch.full((heap.n,), -7, dtype=torch.int64, device="cuda")
    h = u64_to_t(heap.handles, "cuda")
    n_bad = torch.full((1,), -3, dtype=torch.int64, device="cuda")
    m = int(heap.live.sum())
    c_off = torch.empty(m, dtype=torch.int64, device="cuda")
    c_size = torch.empty(m, dtype=torch.int64, device="cuda")
    c_pin = torch.full((m,), 9, dtype=torch.uint8, device="cuda")
    plan, post = ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws, request,
                                   new_off, h, h, n_bad, c_off, c_size, None, c_pin,
                                   tuning=tuning, pinned=pin)
    torch.cuda.synchronize()
    want_pin = (np.zeros(m, np.uint8) if heap.pinned is None
                else heap.pinned[np.flatnonzero(heap.live)])
    assert np.array_equal(c_pin.cpu().numpy(), want_pin)
    return GpuRun(plan, t_to_u64(new_off), t_to_u64(h), int(n_bad.item()), post, 0, arena, ws)


def oracle_arena(heap: W.Heap, hold: Optional[np.ndarray] = None) -> np.ndarray:
    """The whole compacted arena on the host: the generator's pristine
    payload, then the oracle's ordered memmove over it.  Full-size heaps
    need their arena's size in host memory (80 GiB for training-80g)."""
    ref = np.empty(heap.arena_bytes, dtype=np.uint8)
    W.fill_payload(torch.from_numpy(ref), 0, heap.payload_mode, heap.payload_seed)
    oracle.compact(ref, heap.offset, heap.size, heap.live,
                   heap.pinned if hold is None else hold)
    return ref


_libc = None


def check_arena_every_byte(arena: torch.Tensor, ref: np.ndarray, what: str = "",
                           chunk: int = 1 << 30) -> None:
    """Every byte of the device arena against a host arena, chunk by chunk
    through one pinned buffer; reports the first differing bytes."""
    global _libc
    if _libc is None:
        import ctypes
        _libc = ctypes.CDLL(None)
        _libc.memcmp.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
        _libc.memcmp.restype = ctypes.c_int
    S = ref.shape[0]
    assert arena.numel() == S and ref.flags["C_CONTIGUOUS"]
    chunk = min(chunk, max(S, 1))
    buf = torch.empty(chunk, dtype=torch.uint8, pin_memory=True)
    bnp = buf.numpy()
    base = ref.ctypes.data
    for k, p in enumerate(range(0, S, chunk)):
        ln = min(chunk, S - p)
        buf[:ln].copy_(arena[p:p + ln])
        if _libc.memcmp(bnp.ctypes.data, base + p, ln) != 0:
            bad = np.flatnonzero(bnp[:ln] != ref[p:p + ln])
            raise AssertionError(f"{what}: arena differs from the oracle at {bad.shape[0]} bytes "
                                 f"of [{p}, {p + ln}), first {(bad[:8] + p).tolist()}")
        if k % 16 == 15:
            log(f"  {what}: {p + ln} of {S} bytes equal")


def check_stats(got, want, what=""):
    for k in STAT_KEYS:
        g, w = getattr(got, k), getattr(want, k)
        assert g == w, f"{what} stats.{k}: gpu {g} != oracle {w}"


def check_tables_and_handles(heap: W.Heap, r: GpuRun, handles: Optional[np.ndarray] = None,
                             hold: Optional[np.ndarray] = None):
    """new offsets, plan stats, remap, post-move stats: all bit-exact.
    hold: the blocks that stay in place, if not just the pinned ones (a
    targeted plan holds every live block outside its window)."""
    pin = heap.pinned if hold is None else hold
    want_new = oracle.new_offsets(heap.offset, heap.size, heap.live, pin)
    assert np.array_equal(r.new_off, want_new), "new offsets differ"
    check_stats(r.plan.stats, oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes,
                                           pinned=pin), "plan")
    hs = heap.handles if handles is None else handles
    want_h, want_bad = oracle.remap(heap.offset, heap.size, heap.live, hs, pinned=pin)
    assert np.array_equal(r.remapped, want_h), "remapped handles differ"
    assert r.n_invalid == want_bad, (r.n_invalid, want_bad)
    li = np.flatnonzero(heap.live)
    user_pin = heap.pinned
    post_want = oracle.stats(want_new[li], heap.size[li], np.ones(li.shape[0], np.uint8),
                             heap.arena_bytes, pinned=None if user_pin is None else user_pin[li])
    check_stats(r.post_stats, post_want, "post")


def check_arena_full(heap: W.Heap, r: GpuRun, pristine: torch.Tensor,
                     hold: Optional[np.ndarray] = None):
    """Whole arena against the oracle's ordered memmove of the same bytes."""
    ref = pristine.numpy().copy()
    oracle.compact(ref, heap.offset, heap.size, heap.live,
                   heap.pinned if hold is None else hold)
    got = r.arena.cpu().numpy()
    if not np.array_equal(got, ref):
        bad = np.flatnonzero(got != ref)
        raise AssertionError(f"arena differs at {bad.shape[0]} bytes, first {bad[:8].tolist()}")


def sample_windows(heap: W.Heap, rng: np.random.Generator, n_random: int = 2048,
                   win: int = 4096, per_block_cap: int = 4096,
                   hold: Optional[np.ndarray] = None):
    """Windows (start, length) of the compacted arena to check: the first and
    last bytes of (a sample of) every live block at its new place, random
    windows below and above the live total, and the window across it."""
    new = oracle.new_offsets(heap.offset, heap.size, heap.live,
                             heap.pinned if hold is None else hold)
    li = np.flatnonzero(heap.live)
    if li.shape[0] > per_block_cap:
        li = np.sort(rng.choice(li, per_block_cap, replace=False))
    lt = int((heap.size * heap.live).sum())
    S = heap.arena_bytes
    wins = []
    for i in li.tolist():
        a, s = int(new[i]), int(heap.size[i])
        wins.append((a, min(win, s)))
        wins.append((a + s - min(win, s), min(win, s)))
    for p in rng.integers(0, max(S - win, 1), n_random).tolist():
        p = (p // 16) * 16
        wins.append((p, min(win, S - p)))
    if lt > 0 and S > 0:
        p = max(0, lt - win // 2)
        wins.append((p, min(win, S - p)))
    return wins


def check_arena_sampled(heap: W.Heap, r: GpuRun, windows, hold: Optional[np.ndarray] = None):
    """Sampled windows against the oracle's per-byte source map applied to
    the generator's pristine payload."""
    for (p0, ln) in windows:
        if ln <= 0:
            continue
        got = r.arena[p0:p0 + ln].cpu().numpy()
        d, s, l = oracle.source_map(heap.offset, heap.size, heap.live, heap.arena_bytes, p0, ln,
                                    pinned=heap.pinned if hold is None else hold)
        want = np.empty(ln, dtype=np.uint8)
        for dd, ss, ll in zip(d.tolist(), s.tolist(), l.tolist()):
            want[dd - p0:dd - p0 + ll] = W.payload_window(ss, ll, heap.payload_mode,
                                                          heap.payload_seed)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"window [{p0}, {p0 + ln}) differs at {bad[:8].tolist()}")

"""The mover's schedule, read back through defrag_plan_tiles and checked
against one derived on the host from the oracle's new offsets alone.

Bit-exact arena bytes (the other parity tests) show that a move came out
right; they cannot show that no race was possible, since a missing wait may
go unnoticed when the earlier tile happens to load first.  This test checks
the schedule itself: the tiles are exactly the parts of each run of
consecutive moved blocks inside each tile-size window, in ascending order,
with the right blocks and shift, and each tile waits for exactly the earlier
tiles whose source bytes overlap its destination bytes (a tile never needs a
later one, since a byte's source never lies below it).  The plan needs no
arena, so the full-size workloads are checked in their real launch
configuration (64 KiB tiles) as well.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import device_pinned, device_table, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def expected_schedule(heap, hold, T):
    """Tiles (t0, t1, shift_first, first, last, dep_lo, dep_hi) of a plan with
    tile size T, from the oracle's new offsets; hold marks the entries that
    stay in place (pinned, or outside a targeted window).  Empty dependency
    ranges come back as (1, 0)."""
    li = np.flatnonzero(heap.live)
    new = oracle.new_offsets(heap.offset, heap.size, heap.live, hold)[li].astype(np.int64)
    old = heap.offset[li].astype(np.int64)
    sz = heap.size[li].astype(np.int64)
    shift = old - new
    assert np.all(shift >= 0)
    moved = np.flatnonzero(shift > 0)            # packed live-block indices
    if moved.size == 0:
        return np.zeros((0, 7), np.int64)
    ms, me, msh = new[moved], new[moved] + sz[moved], shift[moved]
    assert np.all(me[:-1] <= ms[1:])             # destinations ascend
    # runs: maximal stretches of consecutive moved blocks, packed back to back
    cont = np.diff(moved) == 1
    assert np.array_equal(ms[1:][cont], me[:-1][cont])
    r0 = np.concatenate([[0], np.flatnonzero(~cont) + 1])
    r1 = np.concatenate([np.flatnonzero(~cont), [moved.size - 1]])
    D0, D1 = ms[r0], me[r1]
    # each run cut at every multiple of T
    cnt = (D1 - 1) // T - D0 // T + 1
    run = np.repeat(np.arange(r0.size), cnt)
    j = np.arange(cnt.sum()) - np.repeat(np.cumsum(cnt) - cnt, cnt)
    w0 = D0[run] // T + j
    t0 = np.where(j == 0, D0[run], w0 * T)
    t1 = np.minimum((w0 + 1) * T, D1[run])
    assert np.all(t1 > t0)
    fi = np.searchsorted(me, t0, side="right")   # first moved block ending above t0
    la = np.searchsorted(ms, t1, side="left") - 1  # last one starting below t1
    # source pieces: the common refinement of tiles and moved blocks
    pts = np.unique(np.concatenate([t0, t1, ms, me]))
    a, b = pts[:-1], pts[1:]
    ti = np.searchsorted(t0, a, side="right") - 1
    keep = (ti >= 0) & (a < t1[np.maximum(ti, 0)])
    a, b, ti = a[keep], b[keep], ti[keep]
    bi = np.searchsorted(ms, a, side="right") - 1
    assert np.all(a >= ms[bi]) and np.all(b <= me[bi]) and np.all(b <= t1[ti])
    ps, pe = a + msh[bi], b + msh[bi]
    assert np.all(pe[:-1] <= ps[1:])             # sources ascend too
    first = np.searchsorted(pe, t0, side="right")  # first piece ending above t0
    stop = np.searchsorted(ps, t1, side="left")    # pieces starting below t1
    idx = np.arange(t0.size)
    none = stop <= first                         # bytes that were free before
    owner_lo = ti[np.minimum(first, ti.size - 1)]
    owner_hi = ti[np.maximum(stop - 1, 0)]
    assert np.all(none | (owner_hi <= idx))      # never a later tile
    dep_hi = np.where(owner_hi == idx, idx - 1, owner_hi)
    dep_lo = owner_lo.copy()
    empty = none | (dep_lo > dep_hi)
    dep_lo[empty], dep_hi[empty] = 1, 0
    return np.column_stack([t0, t1, shift[moved[fi]], moved[fi], moved[la], dep_lo, dep_hi])


def auto_tile(heap, hold):
    """The tile size a plan given none must choose, stated on the host: 128 KiB
    in an arena of at most 64 MiB, in a table of small blocks (entries
    averaging under 8 KiB of the arena), or when more than half of the moved
    bytes belong to blocks that shift by less than 8 MiB and at least 64 MiB
    move, else 64 KiB (the workspaces here hold either size's tiles)."""
    if heap.arena_bytes <= (64 << 20) or (heap.n and heap.arena_bytes // heap.n < 8192):
        return 131072
    li = np.flatnonzero(heap.live)
    new = oracle.new_offsets(heap.offset, heap.size, heap.live, hold)[li].astype(np.int64)
    shift = heap.offset[li].astype(np.int64) - new
    sz = heap.size[li].astype(np.int64)
    moved = int(sz[shift > 0].sum())
    small = int(sz[(shift > 0) & (shift < (8 << 20))].sum())
    return 131072 if (2 * small > moved and moved >= (64 << 20)) else 65536


def check_schedule(ac, heap, T=65536, request=0):
    """T None: no tile size given, the plan picks one (checked against the
    rule stated in auto_tile)."""
    hold = heap.pinned
    if request:
        w = oracle.target_window(heap.offset, heap.size, heap.live, heap.arena_bytes, request,
                                 pinned=heap.pinned)
        assert w.found
        hold = oracle.window_pins(heap.offset, heap.live, heap.pinned, w)
    log(f"case schedule {heap.describe()} T={T} request={request}")
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes, T or 0, max_pinned=heap.n_pinned)
    tu = ac.defrag_tuning(T, 0, 1, 0) if T else None   # None: the plan picks the size
    if request:
        plan = ac.defrag_plan_targeted(off, size, live, heap.arena_bytes, request, ws,
                                       tuning=tu, pinned=pin)
    else:
        plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws, tuning=tu, pinned=pin)
    if not T:
        T = auto_tile(heap, hold)
        assert plan.tuning.tile_bytes == T, (plan.tuning.tile_bytes, T)
    got = ac.defrag_plan_tiles(plan, ws)
    want = expected_schedule(heap, hold, T)
    assert got.shape[0] == want.shape[0] == plan.n_tiles, (got.shape, want.shape, plan.n_tiles)
    g = np.column_stack([got[f].astype(np.int64) for f in (
        "dst_begin", "dst_end", "shift_first", "first_block", "last_block", "dep_lo", "dep_hi")])
    g_empty = g[:, 5] > g[:, 6]
    g[g_empty, 5], g[g_empty, 6] = 1, 0
    if not np.array_equal(g, want):
        bad = np.flatnonzero(np.any(g != want, axis=1))
        raise AssertionError(f"{bad.size} tiles differ; first {bad[0]}: gpu {g[bad[0]].tolist()} "
                             f"host {want[bad[0]].tolist()}")
    # whole tiles, as the plan counts them for its workgroup choice
    whole = ((want[:, 1] - want[:, 0]) == T) & (want[:, 3] == want[:, 4])
    assert plan.whole_tiles == int(whole.sum())
    del ws
    return plan


@pytest.mark.parametrize("T", [256, 4096, 65536, 131072, 262144, None])
@pytest.mark.parametrize("k", W.NAMES)
def test_schedule_small_workloads(ac, k, T):
    check_schedule(ac, W.workload(k, small=True), T)


def test_schedule_random_tiny_heaps(ac):
    rng = np.random.default_rng(2024)
    for it in range(40):
        heap = W.tiny_heap(rng, int(rng.integers(1, 400)), sizes=(32, 64, 96, 256, 1024, 4096),
                           gap_p=0.4, pinned_p=0.1 if it % 2 else 0.0)
        check_schedule(ac, heap, int(rng.choice([256, 512, 1024, 4096])))


@pytest.mark.parametrize("T", [4096, 65536])
@pytest.mark.parametrize("m", [2047, 2048, 2049, 2050, 4100])
def test_schedule_at_the_staging_edges(ac, m, T):
    """About 2,048 live blocks, the most a tile-record workgroup stages in
    LDS: every block staged (the searches read LDS alone), one or two more
    (the stretch staged, the blocks past it read from global memory), and
    twice as many.  Blocks of 1 KiB each above a 32-byte hole, so every
    block moves and all form one run: with 4 KiB tiles the tile count falls
    on a multiple of 256 (a workgroup's tiles) at 2,048 blocks and just past
    one above it; with 64 KiB tiles one workgroup's tiles start in more
    blocks than it stages from 2,049 on."""
    s, h = 1024, 32
    blocks = [(h + i * (s + h), s) for i in range(m)]
    S = m * (s + h) + 4096
    heap = W.table_from_lists(S, blocks, [1] * m, name=f"staging edge m={m}")
    plan = check_schedule(ac, heap, T)
    assert plan.n_tiles == -(-m * s // T)  # one run packed from 0, cut at every multiple of T


@pytest.mark.parametrize("k", ["training-80g", "training-80g-pinned"])
def test_schedule_targeted(ac, k):
    heap = W.workload(k, small=True)
    check_schedule(ac, heap, 4096, request=heap.arena_bytes * 42 // 800)


@pytest.mark.parametrize("k", W.NAMES)
def test_schedule_full_size(ac, k):
    """The real launch configuration: full-size tables, the tile size the
    plan picks itself."""
    heap = W.workload(k)
    plan = check_schedule(ac, heap, None)
    log(f"  {plan.n_tiles} tiles, {plan.whole_tiles} whole")
    torch.cuda.empty_cache()


def test_plan_tiles_protocol(ac):
    """A partial copy returns the first tiles; a plan whose workspace was
    planned again is refused (DEFRAG_ENOPLAN), as is a plan from nowhere."""
    import ctypes
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes, 4096)
    tu = ac.defrag_tuning(4096, 0, 1, 0)
    p1 = ac.defrag_plan(off, size, live, heap.arena_bytes, ws, tuning=tu)
    full = ac.defrag_plan_tiles(p1, ws)
    assert full.shape[0] == p1.n_tiles > 8
    part = np.zeros(5, dtype=ac.TILE_DTYPE)
    rc = ac.lib.defrag_plan_tiles(ctypes.byref(p1), ac._ptr(ws), ws.numel(),
                                  ctypes.c_void_p(part.ctypes.data), 5, None)
    assert rc == ac.DEFRAG_OK and np.array_equal(part, full[:5])
    # cap 0 needs no output buffer
    assert ac.lib.defrag_plan_tiles(ctypes.byref(p1), ac._ptr(ws), ws.numel(), None, 0,
                                    None) == ac.DEFRAG_OK
    # a missing output with a non-zero cap
    assert ac.lib.defrag_plan_tiles(ctypes.byref(p1), ac._ptr(ws), ws.numel(), None, 5,
                                    None) == ac.DEFRAG_EINVAL
    p2 = ac.defrag_plan(off, size, live, heap.arena_bytes, ws, tuning=tu)
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_plan_tiles(p1, ws)
    assert e.value.code == ac.DEFRAG_ENOPLAN
    assert np.array_equal(ac.defrag_plan_tiles(p2, ws), full)

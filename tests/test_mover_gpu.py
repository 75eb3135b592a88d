"""The mover's protocol and its failure reports, through the C-ABI:
dependency waits forced with the testing knob (and counted), a tile with
more blocks than the launch holds (DEFRAG_ECAPACITY, not a watchdog), a
workspace overwritten after its plan (DEFRAG_ECORRUPT: no tile outside the
arena moves), statistics of a far larger table beside a plan, and the
one-call path when its plan picks the second tile-size candidate.  Every
condition is forced from the host; every kernel runs to its normal end."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import (check_arena_full, check_tables_and_handles, device_table, log,
                     pristine_host, run_gpu, run_gpu_compact, u64_to_t)

pytestmark = pytest.mark.gpu

MiB = 1 << 20


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def _chained_heap():
    """One 64 MiB block above a 32-byte hole: with 256-byte tiles, tile t + 1
    overwrites the sources of tile t, so every tile but the first waits for
    the one below it."""
    return W.table_from_lists(32 + 64 * MiB, [(0, 32), (32, 64 * MiB)], [0, 1],
                              [40, 4096, 32 + 64 * MiB - 1], name="chained 64 MiB")


def _far_heap():
    """One 256 MiB block above a 64 MiB hole: with 64 KiB tiles, tile t + 1024
    overwrites the sources of tile t -- further back than the tiles in
    flight at once -- so without help almost no tile finds its flag unset."""
    return W.table_from_lists(320 * MiB, [(0, 64 * MiB), (64 * MiB, 256 * MiB)], [0, 1],
                              [64 * MiB, 100 * MiB + 7, 320 * MiB - 1], name="far 256 MiB")


def _report(ac, heap, r):
    rep = ac.defrag_move_report(r.plan, r.ws)
    log(f"  tiles {rep.tiles} late {rep.late_tiles} waited {rep.waited_tiles} polls {rep.polls}")
    assert rep.status == ac.DEFRAG_OK and rep.tiles == r.plan.n_tiles
    assert rep.waited_tiles <= rep.late_tiles <= rep.tiles
    assert (rep.polls == 0) == (rep.waited_tiles == 0)
    return rep


@pytest.mark.parametrize("T", [65536, 131072])
def test_forced_waits_are_counted_and_change_nothing(ac, T):
    """Holding back the flags of some tiles (not of the tiles that depend on
    them, which would sleep as long before looking) makes those dependents
    wait; the counters see it and the bytes do not change.  128 KiB tiles
    are moved two per workgroup in flight, 64 KiB ones one at a time."""
    heap = _far_heap()
    host = pristine_host(heap)
    waited = {}
    n_tiles = 256 * MiB // T
    for every, sleeps in ((0, 0), (16, 64)):
        log(f"case {heap.describe()} tile {T // 1024} KiB, stall every {every} for {sleeps} sleeps")
        tu = ac.defrag_tuning(T, 1, 1, 0, every, sleeps, 99, 0)
        r = run_gpu(heap, tuning=tu, arena=host.cuda())
        assert r.status == ac.DEFRAG_OK and r.plan.n_tiles == n_tiles
        waited[every] = _report(ac, heap, r).waited_tiles
        check_tables_and_handles(heap, r)
        check_arena_full(heap, r, host)
    # n/16 tiles stall for ~0.2 ms; about three in four have a dependent,
    # claimed ~20 us later
    assert waited[16] >= n_tiles // 40 and waited[16] > waited[0]
    # the one-call path reads the same counters
    r = run_gpu_compact(heap, host.cuda(), tuning=ac.defrag_tuning(T, 1, 1, 0, 16, 64, 7, 0))
    assert _report(ac, heap, r).waited_tiles >= n_tiles // 40
    check_tables_and_handles(heap, r)
    check_arena_full(heap, r, host)
    # a heap where every tile waits on the one below it: counters stay
    # consistent and the bytes exact with and without stalls
    heap = _chained_heap()
    host = pristine_host(heap)
    chain_tile = 256 if T == 65536 else T
    for every, sleeps in ((0, 0), (3, 8)):
        log(f"case {heap.describe()} tile {chain_tile}, stall every {every} for {sleeps} sleeps")
        r = run_gpu(heap, tuning=ac.defrag_tuning(chain_tile, 1, 1, 0, every, sleeps, 5, 0),
                    arena=host.cuda())
        assert r.status == ac.DEFRAG_OK
        rep = _report(ac, heap, r)
        # one tile at a time, each finds the one below still loading; two
        # in flight, a tile looks only after the next one's loads went out
        if every or chain_tile == 256:
            assert rep.late_tiles > 0
        check_tables_and_handles(heap, r)
        check_arena_full(heap, r, host)


def test_stall_knob_limits(ac):
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_plan(off, size, live, heap.arena_bytes, ws,
                       tuning=ac.defrag_tuning(0, 1, 1, 0, 1, 4097, 0, 0))
    assert e.value.code == ac.DEFRAG_EINVAL


def test_capacity_is_its_own_error(ac):
    """A tile meeting more blocks than the launch gave it room for stores
    nothing and reports DEFRAG_ECAPACITY (room for one block, forced from
    the host through the plan; the heap's 64 KiB tiles hold several)."""
    heap = W.workload("small-blocks-4g", small=True)
    host = pristine_host(heap)
    arena = host.cuda()
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws)
    assert plan.max_blocks_per_tile > 1 and plan.n_tiles > 0
    plan.max_blocks_per_tile = 1
    ac.defrag_move(arena, plan, ws)
    assert ac.defrag_move_status(plan, ws) == ac.DEFRAG_ECAPACITY
    rep = ac.defrag_move_report(plan, ws)
    assert rep.status == ac.DEFRAG_ECAPACITY
    # the library is unharmed: a fresh plan compacts bit-exactly
    r = run_gpu(heap, arena=host.cuda())
    assert r.status == ac.DEFRAG_OK
    check_arena_full(heap, r, host)


@pytest.mark.parametrize("fill", [0xFF, 0x00])
def test_overwritten_workspace_moves_nothing(ac, fill):
    """Every byte of the workspace after its two headers overwritten between
    plan and move (the headers, and so the plan's epoch, kept): no tile record
    describes bytes inside the arena any more, so the mover stores nothing
    and reports DEFRAG_ECORRUPT."""
    heap = W.workload("training-80g", small=True)
    host = pristine_host(heap)
    arena = host.cuda()
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws)
    assert plan.n_tiles > 0
    ws[512:].fill_(fill)
    torch.cuda.synchronize()
    ac.defrag_move(arena, plan, ws)
    assert ac.defrag_move_status(plan, ws) == ac.DEFRAG_ECORRUPT
    torch.cuda.synchronize()
    assert torch.equal(arena.cpu(), host), "a tile of a damaged plan stored bytes"


def test_statistics_beside_a_plan_of_fewer_entries(ac):
    """defrag_stats and defrag_first_fit write only the workspace's fixed
    statistics region (the scans run on a bounded grid), so a table with
    many more entries than the plan the workspace holds is measured while
    the plan stays intact: it then moves, remaps and commits bit-exactly."""
    small = W.workload("mixed-64m", small=True)
    big = W.workload("small-blocks-4g", small=True)
    assert big.n > 50 * small.n
    host = pristine_host(small)
    arena = host.cuda()
    s_off, s_size, s_live = device_table(small, "cuda")
    b_off, b_size, b_live = device_table(big, "cuda")
    ws = ac.workspace(big.n, max(big.arena_bytes, small.arena_bytes))
    new_off = torch.empty(small.n, dtype=torch.int64, device="cuda")
    plan = ac.defrag_plan(s_off, s_size, s_live, small.arena_bytes, ws, new_off)
    want_big = oracle.stats(big.offset, big.size, big.live, big.arena_bytes)
    st = ac.defrag_stats(b_off, b_size, b_live, big.arena_bytes, ws)
    assert (st.largest_hole, st.hole_count, st.moved_bytes) == \
        (want_big.largest_hole, want_big.hole_count, want_big.moved_bytes)
    R = want_big.largest_hole // 2 + 32
    got, _ = ac.defrag_first_fit(b_off, b_size, b_live, big.arena_bytes, R, ws)
    assert got == oracle.first_fit(big.offset, big.size, big.live, big.arena_bytes, R)
    ac.defrag_move(arena, plan, ws)
    assert ac.defrag_move_status(plan, ws) == ac.DEFRAG_OK
    ref = host.numpy().copy()
    oracle.compact(ref, small.offset, small.size, small.live)
    assert np.array_equal(arena.cpu().numpy(), ref)
    h = ac.defrag_remap(plan, ws, u64_to_t(small.handles, "cuda"))
    m = int(plan.live_blocks)
    c_off = torch.empty(m, dtype=torch.int64, device="cuda")
    ac.defrag_commit(plan, ws, c_off)
    torch.cuda.synchronize()
    want_h, _ = oracle.remap(small.offset, small.size, small.live, small.handles)
    assert np.array_equal(h.cpu().numpy().view(np.uint64), want_h)
    want_new = oracle.new_offsets(small.offset, small.size, small.live)
    assert np.array_equal(c_off.cpu().numpy().view(np.uint64),
                          want_new[np.flatnonzero(small.live)])


def _small_shift_heap():
    """Three 96 MiB blocks above holes of 4 KiB, 64 KiB and 1 MiB and one
    freed 32 MiB block: 288 MiB move, all by less than 8 MiB, so a plan
    given no tile size picks the larger candidate (128 KiB, moved two tiles
    per workgroup in flight)."""
    KiB = 1 << 10
    blocks, live, at = [], [], 0
    for hole, sz in ((4 * KiB, 96 * MiB), (64 * KiB, 96 * MiB), (1 * MiB, 96 * MiB)):
        blocks.append((at, hole))
        live.append(0)
        blocks.append((at + hole, sz))
        live.append(1)
        at += hole + sz
    blocks.append((at, 32 * MiB))
    live.append(0)
    S = at + 32 * MiB
    rng = np.random.default_rng(11)
    handles = np.concatenate([rng.integers(0, S, 4000, dtype=np.uint64),
                              np.array([0, 4 * KiB, 4 * KiB + 96 * MiB - 1, S - 1], np.uint64)])
    return W.table_from_lists(S, blocks, live, handles, name="small shifts 288 MiB")


def test_compact_when_the_plan_picks_the_larger_tile(ac):
    """defrag_compact launches a mover for each tile-size candidate, and the
    remap, commit and post-check run in the first workgroups of the chosen
    one's launch: here the second launch (128 KiB tiles), the first moving
    nothing and running none of them."""
    heap = _small_shift_heap()
    log(f"case compact, plan picks 128 KiB tiles: {heap.describe()}")
    host = pristine_host(heap)
    r = run_gpu_compact(heap, host.cuda())
    assert r.plan.tuning.tile_bytes == 131072
    check_tables_and_handles(heap, r)
    check_arena_full(heap, r, host)

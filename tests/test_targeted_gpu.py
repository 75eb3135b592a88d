"""GPU parity for targeted compaction (defrag_plan_targeted, through the
C-ABI) against the oracle: the chosen window, new offsets, statistics,
remapped handles and the arena bytes, bit-exact.  The oracle's targeted
compaction is its segmented compaction with every live block outside the
oracle's window held in place."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import test_oracle_targeted as TT
from harness import (check_arena_every_byte, check_arena_full, check_arena_sampled,
                     check_tables_and_handles, device_pinned, device_table, log, oracle_arena,
                     pristine_host, run_gpu, sample_windows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def _window_of(plan):
    return (1, plan.window_begin, plan.window_end, plan.window_hole, plan.stats.moved_bytes)


def _check(heap, request, tile=0, full=True, rng=None):
    """One targeted compaction; returns the oracle's window."""
    import arena_compaction_amd as ac
    w = oracle.target_window(heap.offset, heap.size, heap.live, heap.arena_bytes, request,
                             pinned=heap.pinned)
    log(f"case {heap.describe()} request={request} tile={tile} oracle={tuple(w)}")
    tuning = ac.defrag_tuning(tile, 0, 0, 0) if tile else None
    if not w.found:
        _check_nofit(heap, request, tuning)
        return w
    host = pristine_host(heap) if full else None
    r = run_gpu(heap, tuning=tuning, arena=host.cuda() if full else None, request=request)
    assert r.status == ac.DEFRAG_OK, r.status
    assert _window_of(r.plan) == tuple(w), (_window_of(r.plan), tuple(w))
    assert r.plan.request_bytes == request
    hold = oracle.window_pins(heap.offset, heap.live, heap.pinned, w)
    check_tables_and_handles(heap, r, hold=hold)
    if full:
        check_arena_full(heap, r, host, hold=hold)
    else:
        # a full-size heap: windows at the targeted range's edges first, then
        # every byte against the oracle's arena built on the host
        wins = sample_windows(heap, rng, n_random=64, per_block_cap=256, hold=hold)
        top = w.end - w.hole
        for p in (w.begin, max(w.begin, top - 2048), top, max(top, w.end - 4096)):
            wins.append((p, min(4096, heap.arena_bytes - p)))
        check_arena_sampled(heap, r, wins, hold=hold)
        check_arena_every_byte(r.arena, oracle_arena(heap, hold),
                               f"{heap.name} request {request}")
    # the freed hole is there afterwards
    assert r.post_stats.largest_hole >= request
    return w


def _check_nofit(heap, request, tuning):
    import arena_compaction_amd as ac
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes, tuning.tile_bytes if tuning else 0,
                      max_pinned=heap.n_pinned)
    new_off = torch.full((max(heap.n, 1),), -7, dtype=torch.int64, device="cuda")
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_plan_targeted(off, size, live, heap.arena_bytes, request, ws, new_off,
                                tuning=tuning, pinned=pin)
    assert e.value.code == ac.DEFRAG_ENOFIT
    torch.cuda.synchronize()
    assert bool((new_off == -7).all()), "a plan that found no window wrote new offsets"


def test_golden_targeted_gpu(ac):
    for case in TT.golden_cases():
        t = np.array(case["table"], dtype=np.uint64).reshape(-1, 3)
        heap = W.table_from_lists(case["arena_bytes"], [tuple(x) for x in t[:, :2].tolist()],
                                  t[:, 2].tolist(), [], name=case["name"],
                                  pinned=case.get("pinned"))
        heap.handles = W.edge_handles(heap, np.random.default_rng(3), 8)
        for r in case["requests"]:
            for tile in (256, 65536):
                w = _check(heap, r["request"], tile)
                assert list(w) == r["window"]
        c = case.get("compacted")
        if c:
            res = run_gpu(heap, request=c["request"])
            assert res.new_off.tolist() == c["new_offset"]


@pytest.mark.parametrize("tile", (256, 4096, 65536))
def test_random_tiny_heaps_targeted_gpu(ac, tile):
    rng = np.random.default_rng(2000 + tile)
    for k in range(12):
        heap = W.tiny_heap(rng, int(rng.integers(0, 40)), sizes=(32, 64, 96, 160, 1024, 8192),
                           gap_p=float(rng.choice([0.0, 0.3, 0.8])),
                           live_p=float(rng.choice([0.3, 0.6, 0.9, 1.0])),
                           pinned_p=float(rng.choice([0.0, 0.0, 0.2])))
        reqs = TT.requests_for(heap, rng, n_random=3)
        for R in rng.choice(reqs, min(6, len(reqs)), replace=False).tolist():
            _check(heap, int(R), tile)


@pytest.mark.parametrize("k", W.NAMES)
def test_small_workloads_targeted_gpu(ac, k):
    heap = W.workload(k, small=True)
    st_ = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes, pinned=heap.pinned)
    F, L = st_.free_bytes, st_.largest_hole
    for R in sorted({L, L + 1, F // 3, F // 2, F, F + 1}):
        if R >= 1:
            _check(heap, R)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("k", ["training-80g", "training-80g-pinned"])
def test_page_request_full_size(ac, k):
    """The 910C page's 4.2 GB request (4.2/80 of the arena) on the 80 GiB
    workload, and a 4 GiB one that the re-cut gap holds after moving one
    4 KiB block."""
    heap = W.workload(k)
    rng = np.random.default_rng(11)
    for R in (heap.arena_bytes * 42 // 800, 4 * W.GiB):
        w = _check(heap, R, full=False, rng=rng)
        assert w.found and w.moved_bytes < heap.arena_bytes // 16
        torch.cuda.empty_cache()


def test_targeted_edge_cases(ac):
    # empty table: the whole arena is one hole
    heap = W.table_from_lists(4096, [], [], [])
    w = _check(heap, 4096)
    assert tuple(w) == (1, 0, 4096, 4096, 0)
    _check(heap, 4097)
    # nothing free: no request fits
    heap = W.table_from_lists(256, [(0, 128), (128, 128)], [1, 1], [0, 200])
    _check(heap, 1)
    # a request an existing hole holds moves nothing
    heap = W.table_from_lists(1024, [(0, 64), (64, 512), (576, 64)], [1, 0, 1], [10, 600])
    host = pristine_host(heap)
    r = run_gpu(heap, arena=host.cuda(), request=500)
    assert r.plan.n_tiles == 0 and r.plan.stats.moved_bytes == 0
    assert torch.equal(r.arena.cpu(), host)
    # every block live and pinned except one movable block between two holes
    heap = W.table_from_lists(1024, [(0, 64), (128, 64), (256, 64), (512, 64)], [1, 1, 1, 1],
                              [], pinned=[1, 0, 1, 1])
    for R in (64, 128, 192, 193):
        _check(heap, R)


def test_targeted_protocol(ac):
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_plan_targeted(off, size, live, heap.arena_bytes, 0, ws)
    assert e.value.code == ac.DEFRAG_EINVAL
    # an invalid table is reported as such, not as "no fit"
    bad = size.clone()
    bad[3] = 48
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_plan_targeted(off, bad, live, heap.arena_bytes, 4096, ws)
    assert e.value.code == ac.DEFRAG_EINVAL and e.value.invalid_index == 3
    # a targeted call, even one that finds no window, retires an earlier plan
    # in the same workspace: its move then moves nothing
    host = pristine_host(heap)
    arena = host.cuda()
    p1 = ac.defrag_plan(off, size, live, heap.arena_bytes, ws)
    assert p1.n_tiles > 0
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_plan_targeted(off, size, live, heap.arena_bytes, heap.arena_bytes + 32, ws)
    assert e.value.code == ac.DEFRAG_ENOFIT
    ac.defrag_move(arena, p1, ws)
    assert ac.defrag_move_status(p1, ws) == ac.DEFRAG_ENOPLAN
    assert torch.equal(arena.cpu(), host)
    # and a full plan after a targeted one is a normal plan
    big = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes).largest_hole + 32
    p2 = ac.defrag_plan_targeted(off, size, live, heap.arena_bytes, big, ws)
    assert p2.n_tiles > 0   # (a plan with no tiles moves nothing, stale or not)
    p3 = ac.defrag_plan(off, size, live, heap.arena_bytes, ws)
    ac.defrag_move(arena, p2, ws)
    assert ac.defrag_move_status(p2, ws) == ac.DEFRAG_ENOPLAN
    ac.defrag_move(arena, p3, ws)
    assert ac.defrag_move_status(p3, ws) == ac.DEFRAG_OK
    ref = host.numpy().copy()
    oracle.compact(ref, heap.offset, heap.size, heap.live)
    assert np.array_equal(arena.cpu().numpy(), ref)

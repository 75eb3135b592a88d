"""GPU parity for the one-call compaction (defrag_compact): plan, move,
remap, commit and post-check through one C-ABI call, against the oracle,
bit-exact; and its errors leave the arena untouched."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import (check_arena_full, check_stats, check_tables_and_handles,
                     device_pinned, device_table, log, pristine_host, run_gpu_compact, t_to_u64,
                     u64_to_t)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def compact_gpu(heap, arena, request=0, tuning=None):
    return run_gpu_compact(heap, arena, request, tuning)


@pytest.mark.parametrize("k", W.NAMES)
def test_compact_small_workloads(ac, k):
    heap = W.workload(k, small=True)
    log(f"case compact {heap.describe()}")
    host = pristine_host(heap)
    r = compact_gpu(heap, host.cuda())
    check_tables_and_handles(heap, r)
    check_arena_full(heap, r, host)


def test_compact_tiny_heaps_and_tiles(ac):
    """Workgroups per CU 0 (as many as fit: the plain order, plan read back
    before the move) and 1-3 (the move queued behind the plan, sized on the
    device), over tile sizes and nontemporal modes."""
    rng = np.random.default_rng(77)
    for k in range(32):
        heap = W.tiny_heap(rng, int(rng.integers(0, 50)), sizes=(32, 64, 96, 160, 4096),
                           gap_p=float(rng.choice([0.0, 0.3, 0.8])),
                           live_p=float(rng.choice([0.2, 0.6, 1.0])),
                           pinned_p=float(rng.choice([0.0, 0.2])))
        tile = int(rng.choice([256, 4096, 65536]))
        wg = k % 4
        nt = int(rng.integers(0, 4))
        host = pristine_host(heap)
        r = compact_gpu(heap, host.cuda(), tuning=ac.defrag_tuning(tile, wg, nt, 0))
        check_tables_and_handles(heap, r)
        check_arena_full(heap, r, host)


@pytest.mark.parametrize("k", ["training-80g", "training-80g-pinned"])
def test_compact_targeted_small(ac, k):
    heap = W.workload(k, small=True)
    st = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes, pinned=heap.pinned)
    for R in (st.largest_hole + 32, st.free_bytes // 2):
        w = oracle.target_window(heap.offset, heap.size, heap.live, heap.arena_bytes, R,
                                 pinned=heap.pinned)
        assert w.found
        host = pristine_host(heap)
        r = compact_gpu(heap, host.cuda(), request=R)
        assert (r.plan.window_begin, r.plan.window_end, r.plan.window_hole) == \
            (w.begin, w.end, w.hole)
        hold = oracle.window_pins(heap.offset, heap.live, heap.pinned, w)
        check_tables_and_handles(heap, r, hold=hold)
        check_arena_full(heap, r, host, hold=hold)
        assert r.post_stats.largest_hole >= R


def test_compact_errors_leave_the_arena(ac):
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    host = pristine_host(heap)
    arena = host.cuda()
    ws = ac.workspace(heap.n, heap.arena_bytes)
    m = int(heap.live.sum())
    c_off = torch.empty(m, dtype=torch.int64, device="cuda")
    # an invalid table: reported with its entry, nothing moves
    bad = size.clone()
    bad[7] = 40
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, bad, live, heap.arena_bytes, arena, ws, offset_out=c_off,
                          size_out=torch.empty_like(c_off))
    assert e.value.code == ac.DEFRAG_EINVAL and e.value.invalid_index == 7
    # a request no window can free
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws,
                          request_bytes=heap.arena_bytes + 32)
    assert e.value.code == ac.DEFRAG_ENOFIT
    # post-check asked for without the packed table it needs
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws, offset_out=c_off,
                          after=True)
    assert e.value.code == ac.DEFRAG_EINVAL
    # room for fewer tiles than the plan needs (a workspace sized for
    # 128 KiB tiles, planned with 256-byte ones): the plan says so only from
    # the device, and the move queued behind it moves nothing
    ws_few = ac.workspace(heap.n, heap.arena_bytes, 131072)
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws_few,
                          tuning=ac.defrag_tuning(256, 1, 1, 0))
    assert e.value.code == ac.DEFRAG_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(arena.cpu(), host)


def test_compact_failed_plan_after_a_good_one_moves_nothing(ac):
    """The one-call path queues the move before the plan is read back; a
    workspace whose header still holds an earlier plan's tile count must not
    let an invalid table's move run."""
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    host = pristine_host(heap)
    ws = ac.workspace(heap.n, heap.arena_bytes)
    done = host.cuda()
    plan, _ = ac.defrag_compact(off, size, live, heap.arena_bytes, done, ws)
    assert plan.n_tiles > 0
    arena = host.cuda()
    bad = size.clone()
    bad[3] = 0
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, bad, live, heap.arena_bytes, arena, ws)
    assert e.value.code == ac.DEFRAG_EINVAL and e.value.invalid_index == 3
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws,
                          request_bytes=heap.arena_bytes + 32)
    assert e.value.code == ac.DEFRAG_ENOFIT
    torch.cuda.synchronize()
    assert torch.equal(arena.cpu(), host)


def test_plan_stays_usable_after_compact(ac):
    """The one-call path's post-check reuses the workspace's scratch region;
    the plan it returns still reports the move, remaps more handles and
    commits again, also after a statistics pass of a table of the planned
    size on the same workspace."""
    heap = W.workload("training-80g-pinned", small=True)
    log(f"case plan after compact {heap.describe()}")
    host = pristine_host(heap)
    r = compact_gpu(heap, host.cuda())
    check_tables_and_handles(heap, r)
    ws = r.ws
    extra = W.edge_handles(heap, np.random.default_rng(11), 512)
    want_h, want_bad = oracle.remap(heap.offset, heap.size, heap.live, extra, pinned=heap.pinned)
    li = np.flatnonzero(heap.live)
    want_new = oracle.new_offsets(heap.offset, heap.size, heap.live, heap.pinned)[li]
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    for rnd in range(2):
        assert ac.defrag_move_status(r.plan, ws) == ac.DEFRAG_OK
        nb = torch.full((1,), -1, dtype=torch.int64, device="cuda")
        got = ac.defrag_remap(r.plan, ws, u64_to_t(extra, "cuda"), None, nb)
        torch.cuda.synchronize()
        assert np.array_equal(t_to_u64(got), want_h), f"remap differs (pass {rnd})"
        assert int(nb.item()) == want_bad
        c_off = torch.empty(li.shape[0], dtype=torch.int64, device="cuda")
        c_size = torch.empty_like(c_off)
        c_pin = torch.full((li.shape[0],), 9, dtype=torch.uint8, device="cuda")
        ac.defrag_commit(r.plan, ws, c_off, c_size, None, pinned_out=c_pin)
        torch.cuda.synchronize()
        assert np.array_equal(t_to_u64(c_off), want_new)
        assert np.array_equal(t_to_u64(c_size), heap.size[li])
        assert np.array_equal(c_pin.cpu().numpy(), heap.pinned[li])
        # a statistics pass of the original table (as many entries as planned)
        st = ac.defrag_stats(off, size, live, heap.arena_bytes, ws, pinned=pin)
        check_stats(st, oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes,
                                     pinned=heap.pinned), "statistics pass")


@pytest.mark.parametrize("k", ["training-80g", "small-blocks-4g"])
def test_compact_commit_without_post_check(ac, k):
    """The packed table asked for without the post-check (and, separately,
    only its flag columns): commit then runs beside the move on its own,
    and the table it writes is the oracle's."""
    heap = W.workload(k, small=True)
    log(f"case compact commit only {heap.describe()}")
    host = pristine_host(heap)
    off, size, live = device_table(heap, "cuda")
    li = np.flatnonzero(heap.live)
    m = li.shape[0]
    want_new = oracle.new_offsets(heap.offset, heap.size, heap.live, heap.pinned)
    for only_flags in (False, True):
        arena = host.cuda()
        ws = ac.workspace(heap.n, heap.arena_bytes)
        c_off = None if only_flags else torch.empty(m, dtype=torch.int64, device="cuda")
        c_size = None if only_flags else torch.empty(m, dtype=torch.int64, device="cuda")
        c_live = torch.full((m,), 7, dtype=torch.uint8, device="cuda")
        c_pin = torch.full((m,), 9, dtype=torch.uint8, device="cuda")
        plan, post = ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws,
                                       offset_out=c_off, size_out=c_size, live_out=c_live,
                                       pinned_out=c_pin, after=False)
        torch.cuda.synchronize()
        assert post is None and plan.live_blocks == m
        assert bool((c_live == 1).all()) and bool((c_pin == 0).all())
        if not only_flags:
            assert np.array_equal(t_to_u64(c_off), want_new[li])
            assert np.array_equal(t_to_u64(c_size), heap.size[li])
        ref = host.numpy().copy()
        oracle.compact(ref, heap.offset, heap.size, heap.live, heap.pinned)
        assert np.array_equal(arena.cpu().numpy(), ref)


@pytest.mark.parametrize("k", ["mixed-64m", "training-80g"])
def test_compact_side_job_parts(ac, k):
    """Remap, commit and the post-check run in the first workgroups of the
    mover's launch, each only when asked for: handles alone (no packed
    table, no post-check), the invalid-handle count alone (no handles), and
    the packed table with its post-check but no handles -- each against
    the oracle; and after a failed plan none of the caller's outputs is
    written."""
    heap = W.workload(k, small=True)
    log(f"case side job parts {heap.describe()}")
    host = pristine_host(heap)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    m = int(heap.live.sum())
    want_h, want_bad = oracle.remap(heap.offset, heap.size, heap.live, heap.handles)
    want_new = oracle.new_offsets(heap.offset, heap.size, heap.live)
    want_post = oracle.stats(want_new[np.flatnonzero(heap.live)], heap.size[np.flatnonzero(heap.live)],
                             np.ones(m, np.uint8), heap.arena_bytes)
    # handles alone
    h = u64_to_t(heap.handles, "cuda")
    h_out = torch.full_like(h, -5)
    nb = torch.full((1,), -3, dtype=torch.int64, device="cuda")
    plan, post = ac.defrag_compact(off, size, live, heap.arena_bytes, host.cuda(), ws,
                                   handles=h, h_out=h_out, n_invalid=nb)
    assert post is None and plan.live_blocks == m
    assert np.array_equal(t_to_u64(h_out), want_h) and int(nb.item()) == want_bad
    # the count alone: no handles, so nothing is invalid
    nb.fill_(-3)
    ac.defrag_compact(off, size, live, heap.arena_bytes, host.cuda(), ws, n_invalid=nb)
    assert int(nb.item()) == 0
    # the packed table and its post-check, no handles
    c_off = torch.full((m,), -7, dtype=torch.int64, device="cuda")
    c_size = torch.full((m,), -7, dtype=torch.int64, device="cuda")
    c_live = torch.full((m,), 7, dtype=torch.uint8, device="cuda")
    plan, post = ac.defrag_compact(off, size, live, heap.arena_bytes, host.cuda(), ws,
                                   offset_out=c_off, size_out=c_size, live_out=c_live)
    assert np.array_equal(t_to_u64(c_off), want_new[np.flatnonzero(heap.live)])
    assert np.array_equal(t_to_u64(c_size), heap.size[np.flatnonzero(heap.live)])
    assert bool(torch.all(c_live == 1))
    check_stats(post, want_post, "post-check without handles")
    # a failed plan (an invalid entry): no output written
    bad = size.clone()
    bad[1] = 48
    h_out.fill_(-5)
    c_off.fill_(-7)
    c_size.fill_(-7)
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact(off, bad, live, heap.arena_bytes, host.cuda(), ws, handles=h,
                          h_out=h_out, offset_out=c_off, size_out=c_size)
    assert e.value.code == ac.DEFRAG_EINVAL and e.value.invalid_index == 1
    torch.cuda.synchronize()
    assert bool(torch.all(h_out == -5)) and bool(torch.all(c_off == -7))
    assert bool(torch.all(c_size == -7))


@pytest.mark.parametrize("tile", [0, 256])
def test_compact_edge_cases(ac, tile):
    """The one call on degenerate tables -- no entries, nothing live, all
    live with no hole, one tiny block far up -- with every output asked
    for (buffers of at least one entry, so the call takes its one-stream
    path even when nothing is live): new offsets, handles (edges included),
    the packed table, its post-check and every arena byte against the
    oracle."""
    cases = [
        W.table_from_lists(4096, [], [], [0, 5, 4096]),                    # n = 0
        W.table_from_lists(4096, [(0, 1024), (2048, 512)], [0, 0], [0, 2048]),  # all free
        W.table_from_lists(2048, [(0, 1024), (1024, 1024)], [1, 1], [0, 2047]),  # all live, full
        W.table_from_lists(4096, [(0, 1024), (1024, 1024)], [1, 1], [0, 2047, 2048]),
        W.table_from_lists(8192, [(4096, 32)], [1], [4096, 4127]),         # one tiny block
    ]
    tu = ac.defrag_tuning(tile, 1, 1, 0) if tile else None
    for heap in cases:
        log(f"case one-call edge {heap.describe()} tile {tile}")
        host = pristine_host(heap)
        arena = host.cuda()
        off, size, live = device_table(heap, "cuda")
        ws = ac.workspace(max(heap.n, 1), heap.arena_bytes, tile)
        li = np.flatnonzero(heap.live)
        m, k = li.shape[0], max(li.shape[0], 1)
        hs = np.concatenate([heap.handles, W.edge_handles(heap, np.random.default_rng(1), 8)])
        h = u64_to_t(hs, "cuda")
        h_out = torch.full_like(h, -5)
        nb = torch.full((1,), -3, dtype=torch.int64, device="cuda")
        new_off = torch.full((max(heap.n, 1),), -7, dtype=torch.int64, device="cuda")
        c_off = torch.full((k,), -7, dtype=torch.int64, device="cuda")
        c_size = torch.full((k,), -7, dtype=torch.int64, device="cuda")
        c_live = torch.full((k,), 7, dtype=torch.uint8, device="cuda")
        plan, post = ac.defrag_compact(off, size, live, heap.arena_bytes, arena, ws,
                                       new_offset=new_off[:heap.n], handles=h, h_out=h_out,
                                       n_invalid=nb, offset_out=c_off, size_out=c_size,
                                       live_out=c_live, tuning=tu, after=True)
        torch.cuda.synchronize()
        want_new = oracle.new_offsets(heap.offset, heap.size, heap.live)
        assert np.array_equal(t_to_u64(new_off)[:heap.n], want_new)
        want_h, want_bad = oracle.remap(heap.offset, heap.size, heap.live, hs)
        assert np.array_equal(t_to_u64(h_out), want_h) and int(nb.item()) == want_bad
        assert plan.live_blocks == m
        assert np.array_equal(t_to_u64(c_off)[:m], want_new[li])
        assert np.array_equal(t_to_u64(c_size)[:m], heap.size[li])
        assert bool(torch.all(c_live[:m] == 1))
        if m < k:  # nothing live: the packed outputs are not written
            assert int(c_off[0]) == -7 and int(c_size[0]) == -7 and int(c_live[0]) == 7
        want_post = oracle.stats(want_new[li], heap.size[li], np.ones(m, np.uint8),
                                 heap.arena_bytes)
        check_stats(post, want_post, "one-call edge post-check")
        ref = host.numpy().copy()
        oracle.compact(ref, heap.offset, heap.size, heap.live)
        assert np.array_equal(arena.cpu().numpy(), ref)

"""defrag_compact_static -- the one-call compaction for callers that cannot
allocate, on the library's static scratch -- against defrag_compact with a
workspace of the caller's, through the C-ABI: two calls in a row, the second
on a smaller table, each compared field by field and byte by byte (arena,
new offsets, remapped handles, invalid count, packed table, statistics
before and after), and with the oracle.  Then the size limit."""
import numpy as np
import pytest
import torch

import workloads as W
from harness import (check_arena_full, check_tables_and_handles, device_pinned, device_table,
                     log, pristine_host, run_gpu_compact, t_to_u64, u64_to_t)

pytestmark = pytest.mark.gpu

STAT_FIELDS = ("arena_bytes", "live_bytes", "free_bytes", "largest_hole", "hole_count",
               "live_blocks", "moved_blocks", "moved_bytes", "frag_free_over_largest_minus_1",
               "frag_one_minus_largest_over_free", "invalid_index", "invalid_reason")


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def _static_run(ac, heap, arena, request=0):
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    new_off = torch.full((heap.n,), -7, dtype=torch.int64, device="cuda")
    h = u64_to_t(heap.handles, "cuda")
    n_bad = torch.full((1,), -3, dtype=torch.int64, device="cuda")
    m = int(heap.live.sum())
    c_off = torch.empty(m, dtype=torch.int64, device="cuda")
    c_size = torch.empty(m, dtype=torch.int64, device="cuda")
    c_pin = torch.full((m,), 9, dtype=torch.uint8, device="cuda")
    plan, post = ac.defrag_compact_static(off, size, live, heap.arena_bytes, arena, request,
                                          new_off, h, h, n_bad, c_off, c_size, None, c_pin,
                                          pinned=pin)
    torch.cuda.synchronize()
    return plan, post, t_to_u64(new_off), t_to_u64(h), int(n_bad.item()), t_to_u64(c_off), \
        t_to_u64(c_size), c_pin.cpu().numpy()


def test_static_scratch_matches_the_workspace_entry_point(ac):
    # the second call takes a smaller table (fewer entries, a smaller arena)
    cases = [("training-80g-pinned", 0), ("mixed-64m", 0), ("training-80g", 1)]
    sizes = []
    for k, targeted in cases:
        heap = W.workload(k, small=True)
        request = heap.arena_bytes * 42 // 800 if targeted else 0
        log(f"case static scratch {heap.describe()} request={request}")
        host = pristine_host(heap)
        ref = run_gpu_compact(heap, host.cuda(), request=request)
        arena = host.cuda()
        plan, post, new_off, h, n_bad, c_off, c_size, c_pin = _static_run(ac, heap, arena, request)
        for f in STAT_FIELDS:
            assert getattr(plan.stats, f) == getattr(ref.plan.stats, f), f"plan stats.{f}"
            assert getattr(post, f) == getattr(ref.post_stats, f), f"post stats.{f}"
        for f in ("n", "arena_bytes", "live_blocks", "pinned_blocks", "move_begin", "live_bytes",
                  "n_tiles", "whole_tiles", "window_begin", "window_end", "window_hole"):
            assert getattr(plan, f) == getattr(ref.plan, f), f"plan.{f}"
        assert np.array_equal(new_off, ref.new_off)
        assert np.array_equal(h, ref.remapped) and n_bad == ref.n_invalid
        assert torch.equal(arena, ref.arena), "arena bytes differ from defrag_compact's"
        want_off = ref.new_off[np.flatnonzero(heap.live)]
        assert np.array_equal(c_off, want_off) and np.array_equal(c_size,
                                                                 heap.size[heap.live == 1])
        # and against the oracle
        hold = None
        if request:
            import oracle
            w = oracle.target_window(heap.offset, heap.size, heap.live, heap.arena_bytes, request,
                                     pinned=heap.pinned)
            hold = oracle.window_pins(heap.offset, heap.live, heap.pinned, w)
        ref.arena = arena
        check_tables_and_handles(heap, ref, hold=hold)
        check_arena_full(heap, ref, host, hold=hold)
        sizes.append((heap.n, heap.arena_bytes))
        del ref, arena
    assert sizes[1][0] < sizes[0][0] and sizes[1][1] < sizes[0][1]


# the largest mover tile the library takes (a power of two; twice it is
# refused: see test_abi)
MAX_TILE = 262144
TILE_RECORD_BYTES = 52  # a tile's record and flag in the workspace


def test_static_scratch_limits(ac):
    """More tiles than fit beside the plan arrays: refused by the plan on the
    device, before anything moves (a 2^44-byte arena whose one 2^43-byte
    block moves; only the table is read, the arena is never touched).  The
    move needs more tile records than the scratch holds at every tile size
    the plan may pick, so the refusal cannot depend on which it picks.  A
    workspace argument is refused on the host."""
    S = 1 << 44
    assert (S // 2) // MAX_TILE * TILE_RECORD_BYTES > 8 * ac.STATIC_SCRATCH_BYTES
    heap = W.table_from_lists(S, [(0, 1 << 43), (1 << 43, 1 << 43)], [0, 1], [(1 << 43) + 5],
                              name="2^44 arena")
    off, size, live = device_table(heap, "cuda")
    dummy = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_compact_static(off, size, live, S, dummy)
    assert e.value.code == ac.DEFRAG_ETOOBIG
    torch.cuda.synchronize()
    assert int(dummy.sum()) == 0
    # a fitting table right after: the scratch is usable again
    small = W.workload("mixed-64m", small=True)
    host = pristine_host(small)
    ref = run_gpu_compact(small, host.cuda())
    arena = host.cuda()
    plan, post, new_off, h, n_bad, c_off, c_size, c_pin = _static_run(ac, small, arena)
    assert torch.equal(arena, ref.arena) and np.array_equal(new_off, ref.new_off)

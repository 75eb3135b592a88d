"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle,
bit-exact on arena bytes, new offsets, remapped handles and statistics.

Small cases compare every byte; the full-size workloads compare every byte
where the host can hold the arena (mixed-64m, pairs-1g, small-blocks-4g) and otherwise sampled
windows through the oracle's per-byte source map (training-80g, overlap-64g), always with
full new offsets, statistics and handles.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import (check_arena_full, check_arena_sampled, check_stats,
                     check_tables_and_handles, device_table, log, pristine_host, run_gpu,
                     sample_windows, t_to_u64, u64_to_t)

pytestmark = pytest.mark.gpu

TILES = (256, 4096, 65536, 131072, 262144)


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def _tuning(ac, tile=0, wg=0, nt=0):
    return ac.defrag_tuning(tile, wg, nt, 0)


def _full_check(heap, tuning=None, handles=None):
    import arena_compaction_amd as ac
    log(f"case {heap.describe()} tuning={None if tuning is None else (tuning.tile_bytes, tuning.wg_per_cu, tuning.nontemporal)}")
    host = pristine_host(heap)
    r = run_gpu(heap, tuning=tuning, arena=host.cuda(), handles=handles)
    assert r.status == ac.DEFRAG_OK, r.status
    check_tables_and_handles(heap, r, handles)
    check_arena_full(heap, r, host)
    return r


def test_payload_generator_same_on_gpu(ac):
    for mode, seed in (("hash", 0xC0FFEE03), ("counter32", 0x5EED0005)):
        for base in (0, 8 << 30, (1 << 36) + 4096):
            g = torch.empty(3 << 20, dtype=torch.uint8, device="cuda")
            W.fill_payload(g, base, mode, seed, chunk_bytes=1 << 20)
            c = torch.empty(3 << 20, dtype=torch.uint8)
            W.fill_payload(c, base, mode, seed)
            assert torch.equal(g.cpu(), c), (mode, base)


def test_golden_cases_gpu(ac):
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "hand_worked.json")))["cases"]
    for case in cases:
        t = np.array(case["table"], dtype=np.uint64).reshape(-1, 3)
        heap = W.table_from_lists(case["arena_bytes"], [tuple(x) for x in t[:, :2].tolist()],
                                  t[:, 2].tolist(), case["handles"], name=case["name"],
                                  pinned=case.get("pinned"))
        for tile in (256, 65536):
            r = _full_check(heap, _tuning(ac, tile))
            assert r.new_off.tolist() == case["new_offset"]
            want = [W.U64_MAX if v < 0 else v for v in case["remapped"]]
            assert r.remapped.tolist() == want


@pytest.mark.parametrize("tile", TILES)
def test_random_tiny_heaps_gpu(ac, tile):
    rng = np.random.default_rng(1000 + tile)
    for k in range(25):
        n = int(rng.integers(0, 60))
        heap = W.tiny_heap(rng, n, sizes=(32, 64, 96, 160, 4096, 8192),
                           gap_p=float(rng.choice([0.0, 0.3, 0.8])),
                           live_p=float(rng.choice([0.2, 0.5, 0.9, 1.0])),
                           pinned_p=float(rng.choice([0.0, 0.0, 0.15, 0.4])))
        _full_check(heap, _tuning(ac, tile))


def test_random_medium_heaps_default_tuning(ac):
    """Eight seeded heaps of 500-4,000 blocks with sizes log-uniform from 32 B
    to 1 MiB (so shifts range from 32 bytes to many tiles, and tiles mix
    whole single-block windows with many-block ones), varied live, gap and
    pinned fractions, compacted with the library's default tuning (the
    workgroup count the plan picks): every byte, offset and handle against
    the oracle."""
    rng = np.random.default_rng(4242)
    sizes = np.unique((np.exp(rng.uniform(np.log(32), np.log(1 << 20), 96)) // 32 * 32)
                      .astype(np.int64).clip(32))
    for k in range(8):
        n = int(rng.integers(500, 4001))
        heap = W.tiny_heap(rng, n, sizes=tuple(int(x) for x in sizes),
                           gap_p=float(rng.choice([0.0, 0.2, 0.6])),
                           live_p=float(rng.choice([0.3, 0.6, 0.9])),
                           pinned_p=float(rng.choice([0.0, 0.0, 0.02, 0.2])))
        r = _full_check(heap)
        log(f"  tiles {r.plan.n_tiles}, whole {r.plan.whole_tiles}, wg/cu {r.plan.tuning.wg_per_cu}")


@pytest.mark.parametrize("k", W.NAMES)
@pytest.mark.parametrize("tile,nt", [(256, 0), (4096, 1), (65536, 0), (65536, 1), (131072, 0),
                                     (262144, 1)])
def test_small_workloads_gpu(ac, k, tile, nt):
    _full_check(W.workload(k, small=True), _tuning(ac, tile, 0, nt))


@pytest.mark.parametrize("k", ["mixed-64m", "training-80g-pinned", "small-blocks-4g", "overlap-64g"])
def test_one_workgroup_per_cu_and_tiny_tiles(ac, k):
    """Fewer resident workgroups and many more tiles per workgroup: the
    ticket order alone must keep the schedule correct."""
    _full_check(W.workload(k, small=True), _tuning(ac, 512, 1, 0))


def test_tiny_shift_under_large_blocks(ac):
    """One 32-byte hole under a 64 MiB block and a 4 KiB hole under the next:
    every tile's source overlaps its own destination and its successor's."""
    blocks = [(0, 32), (32, 64 << 20), ((64 << 20) + 32, 4096), ((64 << 20) + 4128, 32 << 20)]
    heap = W.table_from_lists((64 << 20) + 4128 + (32 << 20) + 96, blocks, [0, 1, 0, 1],
                              [33, 32 + 12345, (64 << 20) + 4128 + 7])
    for tile in (256, 4096, 65536):
        _full_check(heap, _tuning(ac, tile))


def _chained_heap(tile, lead=0):
    """Live blocks above holes of one tile, one tile + 32 B, two tiles - 32 B
    and three tiles + 32 B (after an optional unmoved live block of `lead`
    bytes): every moved block's source starts at least one tile above its
    destination, and each tile's destination overlaps the source of a tile
    one to three below it."""
    MiB = 1 << 20
    blocks, live, at = [], [], 0
    if lead:
        blocks.append((0, lead)); live.append(1); at = lead
    for hole, n in ((tile, 8 * MiB), (tile + 32, 4 * MiB), (2 * tile - 32, 6 * MiB),
                    (3 * tile + 32, 5 * MiB)):
        blocks.append((at, hole)); live.append(0); at += hole
        blocks.append((at, n)); live.append(1); at += n
    handles = [b[0] + d for b, lv in zip(blocks, live) if lv for d in (0, 4096, b[1] - 1)]
    return W.table_from_lists(at + 4096, blocks, live, handles,
                              name=f"chained tile {tile} lead {lead}")


def test_chained_whole_tiles_without_self_overlap(ac):
    """Whole single-block tiles (the straight-line path) whose source lies at
    least one tile above their destination, each waiting on a tile just below
    it.  With an unmoved 96-byte block first, each block's first and last
    tiles are partial (the general path) and the whole tiles next to them
    wait on them, and the other way round."""
    for tile in (4096, 65536):
        for lead in (0, 96):
            heap = _chained_heap(tile, lead)
            r = _full_check(heap, _tuning(ac, tile))
            if lead == 0:
                assert r.plan.whole_tiles == r.plan.n_tiles, (r.plan.whole_tiles, r.plan.n_tiles)
            else:
                assert 0 < r.plan.whole_tiles < r.plan.n_tiles
            _full_check(heap, _tuning(ac, tile, 1, 1))
    _full_check(_chained_heap(65536, 96))   # library defaults


def test_watchdog_on_chained_whole_tiles_ends_every_wave(ac):
    """A spin limit of two polls on chained whole tiles: whether or not a
    wait gives up, the move returns a status, and the library is bit-exact
    afterwards with the default limit."""
    heap = _chained_heap(4096)
    off, size, live = device_table(heap, "cuda")
    arena = torch.zeros(heap.arena_bytes, dtype=torch.uint8, device="cuda")
    for attempt in range(3):
        log(f"case whole-tile watchdog attempt {attempt}: {heap.describe()} tile 4096, spin limit 2")
        ws = ac.workspace(heap.n, heap.arena_bytes, 4096)
        plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws,
                              tuning=ac.defrag_tuning(4096, 1, 1, 1))
        assert plan.whole_tiles == plan.n_tiles
        ac.defrag_move(arena, plan, ws)
        assert ac.defrag_move_status(plan, ws) in (ac.DEFRAG_OK, ac.DEFRAG_ETIMEOUT)
    del arena
    _full_check(heap, _tuning(ac, 4096, 1, 1))


def test_edge_cases_gpu(ac):
    cases = [
        W.table_from_lists(4096, [], [], [0, 5, 4096]),                    # n = 0
        W.table_from_lists(0, [], [], [0]),                                # empty arena
        W.table_from_lists(4096, [(0, 1024), (2048, 512)], [0, 0], [0, 2048]),  # all free
        W.table_from_lists(2048, [(0, 1024), (1024, 1024)], [1, 1], [0, 2047]),  # all live, full
        W.table_from_lists(4096, [(0, 1024), (1024, 1024)], [1, 1], [0, 2047, 2048]),  # no hole below
        W.table_from_lists(4104, [(32, 4064)], [1], [32, 4095, 4096]),     # ragged 8-byte tail
        W.table_from_lists(8192, [(4096, 32)], [1], [4096, 4127]),         # one tiny block, big shift
    ]
    for heap in cases:
        for tile in (256, 65536):
            r = _full_check(heap, _tuning(ac, tile),
                            handles=np.concatenate([heap.handles,
                                                    W.edge_handles(heap, np.random.default_rng(0), 8)]))
            if heap.live.sum() == 0 or np.all(heap.offset == oracle.new_offsets(
                    heap.offset, heap.size, heap.live)):
                assert r.plan.n_tiles == 0


def test_remap_in_place_and_batches(ac):
    heap = W.workload("pairs-1g", small=True)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws)
    h = u64_to_t(heap.handles, "cuda")
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    ac.defrag_remap(plan, ws, h, h, bad)          # in place, before the move
    want, wb = oracle.remap(heap.offset, heap.size, heap.live, heap.handles)
    assert np.array_equal(t_to_u64(h), want) and int(bad) == wb
    empty = torch.empty(0, dtype=torch.int64, device="cuda")
    ac.defrag_remap(plan, ws, empty, empty, bad)
    assert int(bad) == 0


def test_invalid_tables_gpu(ac):
    """Every validation reason, first failing entry wins, and nothing is
    written: new offsets keep their sentinel, the arena keeps its bytes."""
    U = (1 << 64) - 1
    cases = [
        ([(0, 0, 1)], 64), ([(0, 32, 1), (32, 0, 0)], 64), ([(16, 32, 1)], 64),
        ([(0, 48, 1)], 64), ([(0, 32, 2)], 64), ([(0, 32, 1), (32, 64, 1)], 64),
        ([(96, 32, 1)], 64), ([(0, 64, 1), (32, 32, 0)], 128), ([(64, 32, 1), (0, 32, 1)], 128),
        ([(0, 32, 1), (64, 32, 0), (64, 0, 1)], 128), ([(0, 32, 1), (1 << 63, 1 << 63, 1)], 1 << 63),
        ([(2**64 - 48, 32, 1)], U), ([(2**64 - 32, 32, 1)], U),
    ]
    rng = np.random.default_rng(5)
    # a long valid table with one bad entry deep inside (crosses scan workgroups)
    n = 50_000
    size = np.full(n, 64, np.uint64)
    off = np.arange(n, dtype=np.uint64) * np.uint64(64)
    for bad_at, kind in ((40_000, "overlap"), (2047, "zero"), (2048, "align"), (n - 1, "oob")):
        o, s = off.copy(), size.copy()
        if kind == "overlap":
            o[bad_at] -= np.uint64(32)
        elif kind == "zero":
            s[bad_at] = 0
        elif kind == "align":
            o[bad_at] += np.uint64(16)
        else:
            s[bad_at] = np.uint64(1 << 20)
        cases.append((list(zip(o.tolist(), s.tolist(), rng.integers(0, 2, n).tolist())), n * 64))
    for table, S in cases:
        t = np.array(table, dtype=np.uint64)
        o, s, l = t[:, 0].copy(), t[:, 1].copy(), t[:, 2].astype(np.uint8)
        rc, bad, reason = oracle.validate(o, s, l, S)
        assert rc == oracle.EINVAL
        dev_o, dev_s, dev_l = u64_to_t(o, "cuda"), u64_to_t(s, "cuda"), torch.from_numpy(l).cuda()
        # statistics need partial results only: their workspace ignores the arena size
        ws = ac.workspace(len(table), 1 << 20)
        with pytest.raises(ac.DefragError) as ei:
            ac.defrag_stats(dev_o, dev_s, dev_l, S, ws)
        assert ei.value.code == ac.DEFRAG_EINVAL
        assert (ei.value.invalid_index, ei.value.invalid_reason) == (bad, reason)
        need = ac.defrag_workspace_bytes(len(table), S)
        if need == 0 or need > (256 << 20):
            continue   # planning an arena this size needs a tile table this large
        ws = ac.workspace(len(table), S)
        new = torch.full((len(table),), -7, dtype=torch.int64, device="cuda")
        with pytest.raises(ac.DefragError) as ei:
            ac.defrag_plan(dev_o, dev_s, dev_l, S, ws, new)
        assert ei.value.code == ac.DEFRAG_EINVAL
        assert (ei.value.invalid_index, ei.value.invalid_reason) == (bad, reason)
        assert bool((new == -7).all()), "new offsets written for an invalid table"


def test_plan_protocol_errors(ac):
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    S = heap.arena_bytes
    ws = ac.workspace(heap.n, S)
    arena = torch.empty(S, dtype=torch.uint8, device="cuda")
    W.fill_payload(arena, 0, heap.payload_mode, heap.payload_seed)
    before = arena.clone()
    # workspace too small
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_plan(off, size, live, S, small)
    assert ei.value.code == ac.DEFRAG_EWORKSPACE
    # a stale plan: the workspace was re-planned since -> the mover refuses
    p1 = ac.defrag_plan(off, size, live, S, ws)
    p2 = ac.defrag_plan(off, size, live, S, ws)
    ac.defrag_move(arena, p1, ws)
    assert ac.defrag_move_status(p1, ws) == ac.DEFRAG_ENOPLAN
    torch.cuda.synchronize()
    assert torch.equal(arena, before), "a stale plan moved bytes"
    # wrong arena size
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_move(arena[:-32], p2, ws)
    assert ei.value.code == ac.DEFRAG_EINVAL
    # misaligned arena pointer
    with pytest.raises(ac.DefragError) as ei:
        big = torch.empty(S + 16, dtype=torch.uint8, device="cuda")
        ac.defrag_move(big[8:8 + S], p2, ws)
    assert ei.value.code == ac.DEFRAG_EINVAL
    # the current plan moves once, then is consumed
    ac.defrag_move(arena, p2, ws)
    assert ac.defrag_move_status(p2, ws) == ac.DEFRAG_OK
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_move(arena, p2, ws)
    assert ei.value.code == ac.DEFRAG_ENOPLAN
    ref = before.cpu().numpy().copy()
    oracle.compact(ref, heap.offset, heap.size, heap.live)
    assert np.array_equal(arena.cpu().numpy(), ref)
    # another workspace than the plan's
    ws2 = ac.workspace(heap.n, S)
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_remap(p2, ws2, u64_to_t(heap.handles, "cuda"))
    assert ei.value.code == ac.DEFRAG_ENOPLAN


@pytest.mark.parametrize("k", ["mixed-64m", "pairs-1g", "small-blocks-4g", "small-shift-8g"])
def test_full_size_workloads_every_byte(ac, k):
    heap = W.workload(k)
    _full_check(heap)


def test_pinned_edge_cases_gpu(ac):
    """Pinned blocks at the arena ends, adjacent pinned blocks, everything
    pinned, and runs on both sides of a pinned block inside one tile window
    (so one window holds the end of one run and the start of the next)."""
    cases = [
        W.table_from_lists(4096, [(0, 1024), (1024, 512), (2048, 1024)], [1, 0, 1], [0, 2048, 3071],
                           pinned=[1, 0, 0]),
        W.table_from_lists(4096, [(0, 512), (1024, 512), (3072, 1024)], [1, 1, 1], [600, 1030, 4095],
                           pinned=[0, 0, 1]),
        W.table_from_lists(4096, [(64, 64), (128, 64), (512, 64), (576, 64)], [1, 1, 1, 1],
                           [64, 200, 512, 639], pinned=[1, 1, 1, 1]),
        W.table_from_lists(8192, [(128, 96), (320, 64), (384, 32), (512, 160), (800, 96), (1024, 64)],
                           [1, 1, 1, 1, 1, 1], [130, 330, 390, 600, 801, 1030],
                           pinned=[0, 0, 1, 0, 0, 0]),
        W.table_from_lists(1 << 20, [(4096, 65536), (69632 + 32, 32), (69632 + 4096, 65536),
                                     (200000 // 32 * 32, 64), (262144, 131072)],
                           [1, 1, 1, 1, 1], [5000, 69664, 80000, 262144 + 77],
                           pinned=[0, 1, 0, 1, 0]),
    ]
    for heap in cases:
        for tile in (256, 512, 4096, 65536):
            _full_check(heap, _tuning(ac, tile),
                        handles=np.concatenate([heap.handles,
                                                W.edge_handles(heap, np.random.default_rng(1), 8)]))


def test_pinned_invalid_and_workspace(ac):
    heap = W.table_from_lists(4096, [(0, 1024), (1024, 512)], [0, 1], pinned=[1, 0])
    off, size, live = device_table(heap, "cuda")
    pin = torch.from_numpy(heap.pinned).cuda()
    ws = ac.workspace(2, 4096, max_pinned=2)
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_plan(off, size, live, 4096, ws, pinned=pin)
    assert (ei.value.code, ei.value.invalid_index, ei.value.invalid_reason) == (ac.DEFRAG_EINVAL, 0, 7)
    # a workspace sized for no pinned entries is too small for many small segments
    rng = np.random.default_rng(3)
    n = 4000
    size_np = np.full(n, 64, np.uint64)
    off_np = np.arange(n, dtype=np.uint64) * np.uint64(128)
    live_np = np.ones(n, np.uint8)
    pin_np = (np.arange(n) % 2 == 0).astype(np.uint8)
    big = W.Heap("many_segments", n * 128, off_np, size_np, live_np,
                 np.array([130, 64 * 128 + 70], np.uint64), "hash", 11, 0)
    big.pinned = pin_np
    o, s_, l = device_table(big, "cuda")
    p_ = torch.from_numpy(pin_np).cuda()
    # 64 KiB tiles: room for 11 tiles when nothing is pinned, but 2,000 runs
    small = ac.workspace(n, big.arena_bytes, 65536, max_pinned=0)
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_plan(o, s_, l, big.arena_bytes, small, tuning=_tuning(ac, 65536), pinned=p_)
    assert ei.value.code == ac.DEFRAG_EWORKSPACE
    for tile in (256, 65536):
        _full_check(big, _tuning(ac, tile))


def test_watchdog_turns_a_stalled_wait_into_an_error(ac):
    """Failure handling forced from the host: with a spin limit of two polls,
    tiles that wait on the tile just below them (one 64 MiB block above a
    32-byte hole, 256-byte tiles) give up, and the move reports
    DEFRAG_ETIMEOUT instead of hanging; every wave still exits.  The library
    stays usable: a compaction with the default limit is bit-exact after."""
    MiB = 1 << 20
    heap = W.table_from_lists(32 + 64 * MiB, [(0, 32), (32, 64 * MiB)], [0, 1], [40, 4096])
    off, size, live = device_table(heap, "cuda")
    arena = torch.zeros(heap.arena_bytes, dtype=torch.uint8, device="cuda")
    tripped = False
    for attempt in range(3):
        log(f"case watchdog attempt {attempt}: {heap.describe()} tile 256, spin limit 2 polls")
        ws = ac.workspace(heap.n, heap.arena_bytes, 256)
        plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws,
                              tuning=ac.defrag_tuning(256, 0, 1, 1))
        assert plan.n_tiles == (64 * MiB) // 256   # tile t + 1 waits on tile t
        ac.defrag_move(arena, plan, ws)
        st = ac.defrag_move_status(plan, ws)
        assert st in (ac.DEFRAG_OK, ac.DEFRAG_ETIMEOUT), st
        if st == ac.DEFRAG_ETIMEOUT:
            tripped = True
            break
    assert tripped, "no wait gave up in three moves of 262,145 chained tiles"
    del arena
    _full_check(heap)


def test_remap_in_huge_arenas_with_tiny_tables(ac):
    """A table of a few blocks in an arena of 2^35, 2^36 + 4 KiB, 2^37 - 32,
    2^37 and 2^40 bytes: the remap's buckets are 2^32 to 2^37 bytes wide, so
    its in-bucket search runs on 32-bit keys at the widest bucket they allow
    and on 64-bit offsets above it, and its records are the 8-byte form up
    to the largest arena it holds (old ends up to 2^37 - 32) and the 16-byte
    form from 2^37 on.  Plan and remap only (neither reads the arena); every
    handle matches the oracle."""
    GiB = 1 << 30
    for S in (1 << 35, (1 << 36) + 4096, (1 << 37) - 32, 1 << 37, 1 << 40):
        blocks = [(0, 4096), (GiB, 1 << 20), ((1 << 32) - 4096, 8192), ((1 << 32) + 4096, 4096),
                  (S // 64 * 32, 64 * GiB if S >= (1 << 40) else 32), (S - 4096, 4096)]
        live = [0, 1, 1, 1, 1, 1]
        hs = []
        for o_, sz in blocks:
            for p in (o_, o_ + sz - 1, o_ + sz, o_ + sz // 2):
                for dlt in (-32, -1, 0, 1, 32):
                    if 0 <= p + dlt:
                        hs.append(p + dlt)
        hs += [S - 1, S, (1 << 32) - 1, 1 << 32, (1 << 64) - 1]
        heap = W.table_from_lists(S, blocks, live, hs, name=f"huge S={S}")
        log(f"case {heap.describe()} remap only")
        off, size, lv = device_table(heap, "cuda")
        ws = ac.workspace(heap.n, S, 131072)
        plan = ac.defrag_plan(off, size, lv, S, ws, tuning=ac.defrag_tuning(131072, 0, 1, 0))
        h = torch.from_numpy(heap.handles.view(np.int64)).cuda()
        nb = torch.zeros(1, dtype=torch.int64, device="cuda")
        out = ac.defrag_remap(plan, ws, h, n_invalid=nb)
        torch.cuda.synchronize()
        want, bad = oracle.remap(heap.offset, heap.size, heap.live, heap.handles)
        assert np.array_equal(out.cpu().numpy().view(np.uint64), want) and int(nb) == bad
        del ws


def test_remap_in_a_huge_arena_with_narrow_buckets(ac):
    """64 blocks spread over a 2^38-byte arena: the remap's buckets are 2^31
    bytes wide (32-bit keys) while the arena needs 16-byte records, the one
    combination the tiny tables above do not reach.  Plan and remap only."""
    S = 1 << 38
    step = S // 64
    blocks = [(i * step + (i % 7) * 4096, 4096 * (1 + i % 5)) for i in range(64)]
    live = [i % 3 != 1 for i in range(64)]
    hs = []
    for o_, sz in blocks:
        for p in (o_, o_ + sz - 1, o_ + sz, o_ + sz // 2):
            for dlt in (-32, -1, 0, 1, 32):
                if 0 <= p + dlt:
                    hs.append(p + dlt)
    hs += [S - 1, S, (1 << 37) - 1, 1 << 37, (1 << 64) - 1]
    heap = W.table_from_lists(S, blocks, [int(v) for v in live], hs, name="huge narrow")
    log(f"case {heap.describe()} remap only")
    off, size, lv = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, S, 131072)
    plan = ac.defrag_plan(off, size, lv, S, ws, tuning=ac.defrag_tuning(131072, 0, 1, 0))
    h = torch.from_numpy(heap.handles.view(np.int64)).cuda()
    nb = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = ac.defrag_remap(plan, ws, h, n_invalid=nb)
    torch.cuda.synchronize()
    want, bad = oracle.remap(heap.offset, heap.size, heap.live, heap.handles)
    assert np.array_equal(out.cpu().numpy().view(np.uint64), want) and int(nb) == bad
    del ws


def test_remap_at_bucket_boundaries(ac):
    """Blocks that start and end exactly on power-of-two boundaries, holes
    that span many of them, and handles on every 4 KiB boundary and 16/32
    bytes either side, in arenas whose size is and is not a power of two:
    whatever bucket width the remap index picks, every handle matches the
    oracle."""
    KiB = 1 << 10
    for S, blocks, live in (
            (1 << 20, [(0, 32 * KiB), (64 * KiB, 64 * KiB), (256 * KiB, 4 * KiB),
                       (260 * KiB, 128 * KiB), (512 * KiB, 32), (768 * KiB, 256 * KiB)],
             [1, 0, 1, 1, 1, 1]),
            ((1 << 20) + 96, [(32, 128 * KiB - 32), (128 * KiB, 128 * KiB), (640 * KiB, 32)],
             [1, 1, 1]),
            (3 << 20, [(1 << 20, 1 << 20)], [1])):
        hs = []
        for p in range(0, S + 8 * KiB, 4 * KiB):
            for dlt in (-32, -16, 0, 16, 32):
                if p + dlt >= 0:
                    hs.append(p + dlt)
        hs += [S - 1, S, (1 << 64) - 1]
        heap = W.table_from_lists(S, blocks, live, hs, name=f"buckets S={S}")
        r = _full_check(heap)
        want, bad = oracle.remap(heap.offset, heap.size, heap.live, heap.handles)
        assert np.array_equal(r.remapped, want) and r.n_invalid == bad


def test_remap_index_over_a_dense_cluster(ac):
    """Ten thousand 32-byte live blocks (each above a 32-byte hole) packed
    into the first MiB of a 1 GiB arena, and a few large blocks far above:
    the workgroup that builds the index buckets over the cluster meets more
    live blocks than it stages in LDS, so its lanes search global memory.
    Every handle -- one inside each small block, the large blocks' edges,
    the holes -- matches the oracle, and the arena comes out bit-exact."""
    MiB = 1 << 20
    n_small = 10_000
    blocks = [(32 + 64 * i, 32) for i in range(n_small)]
    blocks += [(256 * MiB, 64 * MiB), (512 * MiB, 128 * MiB), (768 * MiB, 32 * MiB)]
    live = [1] * n_small + [1, 0, 1]
    hs = [32 + 64 * i + 8 * (i % 4) for i in range(n_small)]
    hs += [16 + 64 * i for i in range(0, n_small, 97)]  # holes
    for o, sz in blocks[n_small:]:
        hs += [o - 32, o, o + 32, o + sz - 32, o + sz - 1, o + sz]
    heap = W.table_from_lists(1 << 30, blocks, live, hs, name="dense cluster in 1 GiB")
    r = _full_check(heap)
    want, bad = oracle.remap(heap.offset, heap.size, heap.live, heap.handles)
    assert np.array_equal(r.remapped, want) and r.n_invalid == bad


def test_remap_pass_tails(ac):
    """Each lane of the remap takes handles k, k + stride, ...: handle
    counts that leave the launch's last pass part-filled (1, 3, one past a
    workgroup, one short of a whole pass, one short of and one past four), the handles a random mix of the table's edges and holes,
    in place and into a second buffer; every handle matches the oracle and
    nothing past the last handle is written."""
    heap = W.workload("pairs-1g", small=True)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    plan = ac.defrag_plan(off, size, live, heap.arena_bytes, ws)
    rng = np.random.default_rng(41)
    pool = np.concatenate([heap.handles, W.edge_handles(heap, rng, 4096)])
    lanes = 512 * 256  # the most a standalone remap launch runs
    sentinel = np.uint64(0x5A5A5A5A5A5A5A5A)
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    for H in (1, 3, 257, lanes - 1, 4 * lanes - 1, 4 * lanes + 5):
        hs = pool[rng.integers(0, pool.size, H)]
        want, wb = oracle.remap(heap.offset, heap.size, heap.live, hs)
        h = u64_to_t(hs, "cuda")
        buf = u64_to_t(np.full(H + 64, sentinel, np.uint64), "cuda")
        ac.defrag_remap(plan, ws, h, buf[:H], bad)
        got = t_to_u64(buf)
        assert np.array_equal(got[:H], want) and int(bad) == wb, H
        assert np.all(got[H:] == sentinel), H
        ac.defrag_remap(plan, ws, h, h, bad)  # in place
        assert np.array_equal(t_to_u64(h), want) and int(bad) == wb, H


def test_scan_workgroups_taking_several_steps(ac):
    """Above 1,024 x 1,024 entries each scan workgroup takes several steps of
    1,024 entries with a running carry: 3,000,000 entries of 32-96 bytes with
    random gaps, live flags and a few pinned blocks, compacted bit-exactly at
    two tile sizes, and a bad entry deep inside a later step of a chunk."""
    rng = np.random.default_rng(31)
    n = 3_000_000
    size = (rng.integers(1, 4, n) * 32).astype(np.uint64)
    gap = (rng.integers(0, 3, n) * 32).astype(np.uint64)
    off = np.cumsum(size + gap) - size
    live = (rng.random(n) < 0.55).astype(np.uint8)
    pinned = ((rng.random(n) < 0.002) & (live == 1)).astype(np.uint8)
    S = int(off[-1] + size[-1]) + 4096
    heap = W.Heap("chunked scan 3M", S, off.astype(np.uint64), size, live, np.zeros(0, np.uint64),
                  "hash", 31, 31)
    heap.pinned = pinned
    heap.handles = W.edge_handles(heap, rng, 20_000)
    for tile in (4096, 65536):
        _full_check(heap, _tuning(ac, tile))
    # an overlap in the third step of a later workgroup's chunk (3,000,000
    # entries: 2,930 steps over 977 workgroups of 3 steps, 3,072 entries)
    bad_at = 490 * 3072 + 2 * 1024 + 77
    o = heap.offset.copy()
    o[bad_at] = o[bad_at - 1]
    dev_o, dev_s, dev_l = u64_to_t(o, "cuda"), u64_to_t(size, "cuda"), torch.from_numpy(live).cuda()
    want = oracle.validate(o, size, live, S)
    assert want[0] == oracle.EINVAL
    ws = ac.workspace(n, S)
    with pytest.raises(ac.DefragError) as ei:
        ac.defrag_stats(dev_o, dev_s, dev_l, S, ws)
    assert (ei.value.code, ei.value.invalid_index, ei.value.invalid_reason) == \
        (ac.DEFRAG_EINVAL, want[1], want[2])

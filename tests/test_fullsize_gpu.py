"""Every byte at full size: the three largest heaps -- training-80g (the
80 GiB arena shaped like the 910C page's failure), training-80g-pinned and
overlap-64g -- compacted through the separate calls, through defrag_compact,
and through defrag_compact with the mover's dependency waits forced, each
compared with the oracle on new offsets, statistics, every handle and every
arena byte.

The reference arena is built on the host: the generator's pristine payload,
then the oracle's ordered memmove (the 910C page's "periodic compaction":
each live block moves down by the holes below it, order kept).  The device
arena is streamed back through a pinned buffer and compared chunk by chunk.
These tests need the arena's size in host memory (80 GiB) besides the GPU.

Forced waits: the tuning's testing knob holds back, after its loads, the
"sources read" flag of one tile in 4,096 for about 7 ms -- longer than the
ticket takes to reach the tiles that overwrite its sources, even across the
80 GiB heap's largest shifts -- so those tiles find the flag unset and wait.
The move's report must count such waits, and the bytes must not change.
"""
import gc
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import (check_arena_every_byte, check_arena_sampled, check_tables_and_handles, log,
                     oracle_arena, run_gpu, run_gpu_compact, sample_windows)

pytestmark = pytest.mark.gpu

STALL_EVERY = 4096
STALL_SLEEPS = 2048   # ~7 ms at 2.4 GHz
FULL = ["training-80g", "training-80g-pinned", "overlap-64g"]


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def _fresh_arena(heap):
    arena = torch.empty(heap.arena_bytes, dtype=torch.uint8, device="cuda")
    W.fill_payload(arena, 0, heap.payload_mode, heap.payload_seed)
    torch.cuda.synchronize()
    return arena


def _check_run(heap, r, ref, what, seed):
    check_tables_and_handles(heap, r)
    # a quick look at sampled windows first (names the first bad window)
    check_arena_sampled(heap, r, sample_windows(heap, np.random.default_rng(seed), n_random=64,
                                                per_block_cap=256))
    t0 = time.time()
    check_arena_every_byte(r.arena, ref, what)
    log(f"  {what}: all {heap.arena_bytes} bytes equal ({time.time() - t0:.1f} s)")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("k", FULL)
def test_every_byte_full_size(ac, k):
    heap = W.workload(k)
    log(f"case every byte {heap.describe()}")
    t0 = time.time()
    ref = oracle_arena(heap)
    log(f"  oracle arena built on the host in {time.time() - t0:.1f} s")
    seed = {"training-80g": 3, "training-80g-pinned": 5, "overlap-64g": 5}[k]

    # 1. the separate calls
    arena = _fresh_arena(heap)
    r = run_gpu(heap, arena=arena)
    assert r.status == ac.DEFRAG_OK
    _check_run(heap, r, ref, f"{k} separate calls", seed)
    if k.startswith("training-80g"):
        assert abs(r.plan.stats.frag_free_over_largest_minus_1 - 4.7) < 1e-3
        if k == "training-80g":
            assert r.post_stats.hole_count == 1 and r.post_stats.frag_free_over_largest_minus_1 == 0
        else:   # the pinned blocks keep free space in separate holes
            assert 1 < r.post_stats.hole_count and 0 < r.post_stats.frag_free_over_largest_minus_1
    del r, arena
    torch.cuda.empty_cache()

    # 2. one call
    r = run_gpu_compact(heap, _fresh_arena(heap))
    _check_run(heap, r, ref, f"{k} one call", seed + 1)
    rep = ac.defrag_move_report(r.plan, r.ws)
    assert rep.status == ac.DEFRAG_OK and rep.tiles == r.plan.n_tiles
    log(f"  {k} one call: {rep.tiles} tiles, {rep.late_tiles} late, {rep.waited_tiles} waited, "
        f"{rep.polls} polls")
    del r, rep
    torch.cuda.empty_cache()

    # 3. one call with the waits forced
    tu = ac.defrag_tuning(0, 1, 1, 0, STALL_EVERY, STALL_SLEEPS, 1000 + seed, 0)
    r = run_gpu_compact(heap, _fresh_arena(heap), tuning=tu)
    rep = ac.defrag_move_report(r.plan, r.ws)
    log(f"  {k} forced waits: {rep.tiles} tiles, {rep.late_tiles} late, {rep.waited_tiles} "
        f"waited, {rep.polls} polls")
    assert rep.status == ac.DEFRAG_OK
    assert rep.waited_tiles > 0 and rep.polls > 0, "no tile waited with the flags held back"
    _check_run(heap, r, ref, f"{k} forced waits", seed + 2)
    del r, ref
    gc.collect()
    torch.cuda.empty_cache()

"""Read-backs: every call that returns figures ends by copying a result
header into a pinned host slot taken from a shared pool and polling for its
sequence number.  Calls from several host threads at once each get their
own slot and their own header; a long call (its move runs past the polling
window) ends in the blocking wait and reads the same header."""
import threading

import pytest
import torch

import oracle
import workloads as W
from harness import (U64_MAX, check_arena_full, check_stats, check_tables_and_handles,
                     device_table, log, pristine_host, run_gpu_compact)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def test_statistics_from_threads_at_once(ac):
    """Four threads, each with its own table, workspace and stream, call
    defrag_stats and defrag_first_fit 40 times each; every answer is its
    own table's."""
    kinds = ("mixed-64m", "small-blocks-4g", "training-80g", "pairs-1g")
    jobs = []
    for k in kinds:
        heap = W.workload(k, small=True)
        want = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes,
                            pinned=heap.pinned)
        R = want.largest_hole // 2 + 32
        fit = oracle.first_fit(heap.offset, heap.size, heap.live, heap.arena_bytes, R)
        fit = None if fit == U64_MAX else fit
        jobs.append((heap, want, R, fit))
    errors = []

    def work(heap, want, R, fit):
        try:
            torch.cuda.set_device(0)
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                off, size, live = device_table(heap, "cuda")
                pinned = None if heap.pinned is None else torch.from_numpy(heap.pinned).cuda()
                ws = ac.workspace(heap.n, heap.arena_bytes)
                stream.synchronize()
                for _ in range(40):
                    st = ac.defrag_stats(off, size, live, heap.arena_bytes, ws, stream=stream,
                                         pinned=pinned)
                    check_stats(st, want, heap.name)
                    got, _ = ac.defrag_first_fit(off, size, live, heap.arena_bytes, R, ws,
                                                 stream=stream, pinned=pinned)
                    assert got == fit, (heap.name, got, fit)
        except BaseException as e:  # reported by the main thread
            errors.append((heap.name, repr(e)))

    threads = [threading.Thread(target=work, args=j) for j in jobs]
    log(f"case {len(threads)} threads: " + ", ".join(j[0].describe() for j in jobs))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


def test_long_call_ends_in_the_blocking_wait(ac):
    """A compaction whose move takes milliseconds outlasts the polling
    window: the call then blocks on its stream and still returns the plan's
    and the post-check's headers."""
    heap = W.workload("training-80g", small=True)
    host = pristine_host(heap)
    log(f"case long one-call compaction {heap.describe()}")
    r = run_gpu_compact(heap, host.cuda())
    check_tables_and_handles(heap, r)
    check_arena_full(heap, r, host)

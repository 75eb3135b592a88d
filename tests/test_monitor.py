"""The library's layout monitor (defrag_monitor, host arithmetic behind the
C-ABI) against the oracle's, on the hand-worked cases and on random
statistics; its argument errors; and, on the GPU, on statistics that
defrag_stats measured before and after a targeted compaction."""
import ctypes
import math

import numpy as np
import pytest

import oracle
import test_oracle_monitor as MO

U64_MAX = (1 << 64) - 1


def _stats(ac, S, live, largest):
    st = ac.defrag_stats_t()
    F = S - live
    st.arena_bytes, st.live_bytes, st.free_bytes, st.largest_hole = S, live, F, largest
    # what defrag_stats reports for these figures (its documented formulas)
    st.frag_free_over_largest_minus_1 = F / largest - 1.0 if F else 0.0
    st.frag_one_minus_largest_over_free = 1.0 - largest / F if F else 0.0
    st.invalid_index = U64_MAX
    return st


def _run_lib(S, live, largest, warn, crit, tau, req, growth):
    import arena_compaction_amd as ac
    return ac.defrag_monitor(_stats(ac, S, live, largest), warn, crit, tau, req, growth)


def _same(a, b):
    assert a.level == b.level and a.action == b.action
    assert a.usage_ratio == b.usage_ratio
    assert a.frag_free_over_largest_minus_1 == b.frag_free_over_largest_minus_1
    assert a.seconds_to_full == b.seconds_to_full or (
        math.isinf(a.seconds_to_full) and math.isinf(b.seconds_to_full))


@pytest.mark.parametrize("case", MO.golden_cases(), ids=lambda c: c["name"])
def test_library_golden(case):
    MO.check_case(case, _run_lib)


def test_library_matches_oracle_random():
    rng = np.random.default_rng(23)
    for _ in range(4000):
        S = int(rng.integers(1, 1 << 44))
        live = int(rng.integers(0, S + 1))
        F = S - live
        largest = int(rng.integers(1, F + 1)) if F else 0
        req = int(rng.choice([0, int(rng.integers(1, 2 * S + 64)), U64_MAX - int(rng.integers(0, 40))]))
        tau = float(rng.choice([0.0, -1.0, rng.uniform(0, 10)]))
        g = float(rng.choice([0.0, -1.0, rng.uniform(1, 1e9)]))
        w, c = sorted(rng.uniform(0, 1, 2).tolist())
        _same(_run_lib(S, live, largest, w, c, tau, req, g),
              oracle.monitor(S, live, largest, w, c, tau, req, g))


def test_library_argument_errors():
    import arena_compaction_amd as ac
    L = ac.lib
    st = _stats(ac, 1 << 20, 1 << 19, 1 << 18)
    out = ac.defrag_monitor_report()
    assert L.defrag_monitor(None, None, ctypes.byref(out)) == ac.DEFRAG_EINVAL
    assert L.defrag_monitor(ctypes.byref(st), None, None) == ac.DEFRAG_EINVAL
    assert L.defrag_monitor(ctypes.byref(st), None, ctypes.byref(out)) == ac.DEFRAG_OK
    assert out.level == 0 and out.action == 0
    bad = _stats(ac, 1 << 20, 1 << 19, 1 << 18)
    bad.invalid_reason = 5
    assert L.defrag_monitor(ctypes.byref(bad), None, ctypes.byref(out)) == ac.DEFRAG_EINVAL
    bad = _stats(ac, 1 << 20, 1 << 19, 1 << 18)
    bad.largest_hole = (1 << 19) + 32        # larger than the free total
    assert L.defrag_monitor(ctypes.byref(bad), None, ctypes.byref(out)) == ac.DEFRAG_EINVAL
    cfg = ac.defrag_monitor_cfg(float("nan"), 0.95, 0.0, 0, 0.0)
    assert L.defrag_monitor(ctypes.byref(st), ctypes.byref(cfg), ctypes.byref(out)) == ac.DEFRAG_EINVAL


@pytest.mark.gpu
@pytest.mark.parametrize("k", ["training-80g", "training-80g-pinned"])
def test_monitor_on_measured_stats_gpu(k):
    """The 910C story on the GPU: the monitor asks for a targeted compaction
    for the 4.2 GB request, and for nothing once it has run."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd as ac
    import workloads as W
    from harness import device_pinned, device_table, log, run_gpu
    heap = W.workload(k)
    S = heap.arena_bytes
    R = S * 42 // 800
    log(f"case {heap.describe()} monitor before/after targeted compaction for {R}")
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, S, max_pinned=heap.n_pinned)
    st = ac.defrag_stats(off, size, live, S, ws, pinned=device_pinned(heap, "cuda"))
    got = ac.defrag_monitor(st, frag_threshold=4.0, next_request=R)
    o = oracle.stats(heap.offset, heap.size, heap.live, S, pinned=heap.pinned)
    want = oracle.monitor(S, o.live_bytes, o.largest_hole, 0.85, 0.95, 4.0, R, 0.0)
    _same(got, want)
    assert ac.ACTIONS[got.action] == "targeted"
    del ws
    r = run_gpu(heap, request=-(-R // 32) * 32)
    after = ac.defrag_monitor(r.post_stats, frag_threshold=4.0, next_request=R)
    assert ac.ACTIONS[after.action] == "none"
    torch.cuda.empty_cache()

"""GPU parity for first fit (defrag_first_fit, through the C-ABI) against the
oracle, and the allocation proof on the GPU: a request first fit refuses
before a targeted compaction is placed, after it, on the table that
defrag_commit writes, exactly where the oracle places it."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import test_oracle_first_fit as FF
import test_oracle_targeted as TT
from harness import device_pinned, device_table, log, run_gpu, u64_to_t

pytestmark = pytest.mark.gpu
U64_MAX = (1 << 64) - 1


@pytest.fixture(scope="module")
def ac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import arena_compaction_amd
    return arena_compaction_amd


def _gpu_first_fit(ac, off, size, live, S, R, ws, pinned=None):
    got, st = ac.defrag_first_fit(off, size, live, S, R, ws, pinned=pinned)
    return U64_MAX if got is None else got, st


def _check_heap(ac, heap, requests):
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes, max_pinned=heap.n_pinned)
    want_st = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes, pinned=heap.pinned)
    for R in requests:
        want = oracle.first_fit(heap.offset, heap.size, heap.live, heap.arena_bytes, R)
        got, st = _gpu_first_fit(ac, off, size, live, heap.arena_bytes, R, ws, pin)
        assert got == want, (heap.describe(), R, got, want)
        assert st.largest_hole == want_st.largest_hole and st.hole_count == want_st.hole_count


def _after_targeted(ac, heap, request):
    """Targeted compaction on the GPU, then the committed table as tensors."""
    r = run_gpu(heap, request=request)
    m = int(r.plan.live_blocks)
    c_off = torch.empty(m, dtype=torch.int64, device="cuda")
    c_size = torch.empty(m, dtype=torch.int64, device="cuda")
    ac.defrag_commit(r.plan, r.ws, c_off, c_size, None)
    return r, c_off, c_size


def test_golden_first_fit_gpu(ac):
    for case in TT.golden_cases():
        ff = case.get("first_fit")
        if not ff:
            continue
        off, size, live, pin = TT._table(case)
        heap = W.table_from_lists(case["arena_bytes"], list(zip(off.tolist(), size.tolist())),
                                  live.tolist(), [], pinned=None if pin is None else pin.tolist())
        g_off, g_size, g_live = device_table(heap, "cuda")
        ws = ac.workspace(heap.n, heap.arena_bytes, max_pinned=heap.n_pinned)
        for R, want in ff["before"]:
            assert _gpu_first_fit(ac, g_off, g_size, g_live, heap.arena_bytes, R, ws)[0] == want
        if "after" in ff:
            r, c_off, c_size = _after_targeted(ac, heap, ff["after"]["request"])
            for R, want in ff["after"]["expect"]:
                got = _gpu_first_fit(ac, c_off, c_size, None, heap.arena_bytes, R, r.ws)[0]
                assert got == want, (R, got, want)


def test_random_tiny_heaps_first_fit_gpu(ac):
    rng = np.random.default_rng(31)
    for k in range(30):
        heap = W.tiny_heap(rng, int(rng.integers(0, 50)), sizes=(32, 64, 96, 160, 1024, 8192),
                           gap_p=float(rng.choice([0.0, 0.3, 0.8])),
                           live_p=float(rng.choice([0.3, 0.6, 0.9, 1.0])),
                           pinned_p=float(rng.choice([0.0, 0.2])))
        _check_heap(ac, heap, FF.requests_for(heap, rng))
    # arena sizes that are not multiples of 32: only the tail shows the rounding
    for S, reqs in ((120, (24, 32, 33, 56)), (100, (1, 36, 37))):
        heap = W.table_from_lists(S, [(0, 64)], [1])
        _check_heap(ac, heap, reqs)


@pytest.mark.parametrize("k", W.NAMES)
def test_small_workloads_first_fit_gpu(ac, k):
    heap = W.workload(k, small=True)
    st_ = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes, pinned=heap.pinned)
    L, F = st_.largest_hole, st_.free_bytes
    _check_heap(ac, heap, sorted({1, 32, L - 31 if L > 31 else 1, L, L + 1, F, F + 1}))


@pytest.mark.parametrize("k", ["training-80g", "training-80g-pinned"])
def test_allocation_proof_full_size(ac, k):
    """The 910C page's 4.2 GB buffer on the 80 GiB workload: refused before,
    placed after the targeted compaction, where the oracle places it."""
    heap = W.workload(k)
    S = heap.arena_bytes
    R = S * 42 // 800
    log(f"case {heap.describe()} first fit of {R} before and after targeted compaction")
    off, size, live = device_table(heap, "cuda")
    pin = device_pinned(heap, "cuda")
    ws = ac.workspace(heap.n, S, max_pinned=heap.n_pinned)
    assert _gpu_first_fit(ac, off, size, live, S, R, ws, pin)[0] == U64_MAX
    del ws
    r, c_off, c_size = _after_targeted(ac, heap, FF.ceil32(R))
    got = _gpu_first_fit(ac, c_off, c_size, None, S, R, r.ws)[0]
    w = oracle.target_window(heap.offset, heap.size, heap.live, S, FF.ceil32(R),
                             pinned=heap.pinned)
    assert got == w.end - w.hole == r.plan.window_end - r.plan.window_hole
    torch.cuda.empty_cache()


def test_first_fit_invalid_table(ac):
    heap = W.workload("mixed-64m", small=True)
    off, size, live = device_table(heap, "cuda")
    ws = ac.workspace(heap.n, heap.arena_bytes)
    bad = off.clone()
    bad[5] = bad[4]   # overlaps entry 4
    with pytest.raises(ac.DefragError) as e:
        ac.defrag_first_fit(bad, size, live, heap.arena_bytes, 64, ws)
    assert e.value.code == ac.DEFRAG_EINVAL and e.value.invalid_index == 5
    assert e.value.invalid_reason == 5

"""Pins for the oracle's first fit (oracle_first_fit, the CANN page's pool of
section 2.2 on a table) and for the allocation proof that ties it to
targeted compaction:

* hand-worked expectations before and after a targeted compaction
  (tests/golden/targeted_hand_worked.json);
* the pool run on byte maps (tests/bruteforce.py), exhaustively over every
  live mask of small tables and on random tiny heaps;
* the proof itself: a request first fit refuses is placed after a targeted
  compaction for its rounded size whenever that compaction finds a window,
  exactly at the freed hole; and never when it does not.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import workloads as W
import bruteforce as BF
import test_oracle_targeted as TT

U64_MAX = (1 << 64) - 1


def ceil32(x):
    return -(-x // 32) * 32


def check_golden():
    for case in TT.golden_cases():
        ff = case.get("first_fit")
        if not ff:
            continue
        off, size, live, pin = TT._table(case)
        S = case["arena_bytes"]
        for R, want in ff["before"]:
            assert oracle.first_fit(off, size, live, S, R) == want, (R, want)
        if "after" not in ff:
            continue
        w = oracle.target_window(off, size, live, S, ff["after"]["request"], pinned=pin)
        hold = oracle.window_pins(off, live, pin, w)
        new = oracle.new_offsets(off, size, live, hold)
        li = np.flatnonzero(live)
        ones = np.ones(li.shape[0], np.uint8)
        for R, want in ff["after"]["expect"]:
            assert oracle.first_fit(new[li], size[li], ones, S, R) == want, (R, want)


def test_golden_first_fit(oracle_lib):
    check_golden()


def requests_for(heap, rng):
    rs = set(TT.requests_for(heap, rng, n_random=4))
    rs |= {max(1, r - 31) for r in list(rs)}   # values that round up to the same size
    return sorted(rs)


def check_against_bruteforce(heap, rng):
    S = heap.arena_bytes
    for R in requests_for(heap, rng):
        got = oracle.first_fit(heap.offset, heap.size, heap.live, S, R)
        assert got == BF.first_fit(S, heap.offset, heap.size, heap.live, R), R


def check_proof(heap, rng):
    """First fit after targeted compaction for the rounded request."""
    S = heap.arena_bytes
    li = np.flatnonzero(heap.live)
    ones = np.ones(li.shape[0], np.uint8)
    for R in requests_for(heap, rng):
        before = oracle.first_fit(heap.offset, heap.size, heap.live, S, R)
        w = oracle.target_window(heap.offset, heap.size, heap.live, S, ceil32(R),
                                 pinned=heap.pinned)
        if before != U64_MAX:
            # a hole already holds it: the window is that hole, nothing moves
            assert w.found and w.moved_bytes == 0 and w.begin == before
            continue
        if not w.found:
            continue
        hold = oracle.window_pins(heap.offset, heap.live, heap.pinned, w)
        new = oracle.new_offsets(heap.offset, heap.size, heap.live, hold)
        after = oracle.first_fit(new[li], heap.size[li], ones, S, R)
        assert after == w.end - w.hole, (R, after, tuple(w))


def test_exhaustive_live_masks(oracle_lib):
    blocks = [(32, 32), (64, 64), (160, 96), (256, 32), (320, 64)]
    rng = np.random.default_rng(5)
    for tail in (0, 96, 100):   # 100: an arena size that is not a multiple of 32
        S = 384 + tail
        for states in itertools.product((0, 1, 2), repeat=len(blocks)):
            live = [1 if x else 0 for x in states]
            pin = [1 if x == 2 else 0 for x in states]
            heap = W.table_from_lists(S, blocks, live, pinned=pin)
            check_against_bruteforce(heap, rng)
            check_proof(heap, rng)


@settings(max_examples=120, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**32 - 1), n=st.integers(0, 30),
       gap_p=st.sampled_from([0.0, 0.3, 0.8]), live_p=st.sampled_from([0.0, 0.5, 0.9, 1.0]),
       pinned_p=st.sampled_from([0.0, 0.2]))
def test_random_tiny_heaps_first_fit(seed, n, gap_p, live_p, pinned_p):
    rng = np.random.default_rng(seed)
    heap = W.tiny_heap(rng, n, sizes=(32, 64, 96, 160, 1024), gap_p=gap_p, live_p=live_p,
                       pinned_p=pinned_p)
    check_against_bruteforce(heap, rng)
    check_proof(heap, rng)


def test_request_validation(oracle_lib):
    off = np.array([0], np.uint64)
    size = np.array([64], np.uint64)
    live = np.array([0], np.uint8)
    with pytest.raises(ValueError):
        oracle.first_fit(off, size, live, 64, 0)
    with pytest.raises(ValueError):
        oracle.first_fit(off, size, live, 64, U64_MAX - 30)
    assert oracle.first_fit(off, size, live, 64, U64_MAX - 31) == U64_MAX


def test_page_failure_and_proof_on_training_80g(oracle_lib):
    """910C page: with 14 GB free and the largest block under 3 GB, the
    4.2 GB buffer cannot be allocated; after the targeted compaction it is
    placed at the hole that compaction freed."""
    heap = W.workload("training-80g")
    S = heap.arena_bytes
    R = S * 42 // 800
    assert oracle.first_fit(heap.offset, heap.size, heap.live, S, R) == U64_MAX
    w = oracle.target_window(heap.offset, heap.size, heap.live, S, ceil32(R))
    hold = oracle.window_pins(heap.offset, heap.live, None, w)
    new = oracle.new_offsets(heap.offset, heap.size, heap.live, hold)
    li = np.flatnonzero(heap.live)
    got = oracle.first_fit(new[li], heap.size[li], np.ones(li.shape[0], np.uint8), S, R)
    assert got == w.end - w.hole

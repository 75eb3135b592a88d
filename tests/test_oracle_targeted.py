"""Pins for the oracle's targeted compaction (oracle_target_window), against
things other than the oracle itself:

* layouts worked by hand (tests/golden/targeted_hand_worked.json, cited);
* a byte-map simulation that tries every window (tests/bruteforce.py),
  exhaustively over every free/live/pinned assignment of small tables and on
  random tiny heaps, for requests at and around every hole size;
* properties fixed by the definition: the window frees at least the request
  in one piece and moves exactly its live bytes; a request fits iff it fits
  after a full compaction; a larger request never moves fewer bytes.
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import workloads as W
import bruteforce as BF

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_cases():
    with open(os.path.join(HERE, "golden", "targeted_hand_worked.json")) as f:
        return json.load(f)["cases"]


def _table(case):
    t = np.array(case["table"], dtype=np.uint64).reshape(-1, 3)
    pin = np.array(case["pinned"], dtype=np.uint8) if "pinned" in case else None
    return t[:, 0].copy(), t[:, 1].copy(), t[:, 2].astype(np.uint8), pin


def check_golden(case):
    off, size, live, pin = _table(case)
    S = case["arena_bytes"]
    for r in case["requests"]:
        got = oracle.target_window(off, size, live, S, r["request"], pinned=pin)
        assert list(got) == r["window"], (case["name"], r)
    for r in case.get("unpinned_requests", []):
        got = oracle.target_window(off, size, live, S, r["request"], pinned=None)
        assert list(got) == r["window"], (case["name"], r)
    c = case.get("compacted")
    if c:
        w = oracle.target_window(off, size, live, S, c["request"], pinned=pin)
        fixed = oracle.window_pins(off, live, pin, w)
        new = oracle.new_offsets(off, size, live, fixed)
        assert new.tolist() == c["new_offset"]
        li = np.flatnonzero(live)
        assert [[int(new[i]), int(size[i])] for i in li] == c["after_live"]
        post = oracle.stats(new[li], size[li], np.ones(li.shape[0], np.uint8), S)
        assert post.largest_hole == c["after_largest_hole"]
        assert post.hole_count == c["after_hole_count"]


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_golden_targeted(case, oracle_lib):
    check_golden(case)


def requests_for(heap, rng, n_random=6):
    """At and around every hole size, every sum of neighbouring holes, the
    free total, plus a few random byte counts (not only multiples of 32)."""
    st_ = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes)
    B = BF.live_bitmap(heap.arena_bytes, heap.offset, heap.size, heap.live)
    hs = [h[1] for h in BF.holes(B)]
    rs = {1, 32}
    for i in range(len(hs)):
        acc = 0
        for j in range(i, min(len(hs), i + 4)):
            acc += hs[j]
            rs.update((acc - 1, acc, acc + 1))
    rs.update((st_.free_bytes, st_.free_bytes + 1))
    if st_.free_bytes > 1:
        rs.update(int(x) for x in rng.integers(1, st_.free_bytes + 64, n_random))
    return sorted(r for r in rs if r >= 1)


def check_against_bruteforce(heap, rng):
    S = heap.arena_bytes
    for R in requests_for(heap, rng):
        got = tuple(oracle.target_window(heap.offset, heap.size, heap.live, S, R,
                                         pinned=heap.pinned))
        want = BF.target_window(S, heap.offset, heap.size, heap.live, R, heap.pinned)
        assert got == want, (R, got, want)


def test_exhaustive_states_and_requests(oracle_lib):
    """Every (free, live, pinned) assignment of a 5-entry table with gaps,
    every request at and around the hole sizes."""
    blocks = [(32, 32), (64, 64), (160, 96), (256, 32), (320, 64)]
    rng = np.random.default_rng(7)
    for tail in (0, 96):
        S = 384 + tail
        for states in itertools.product((0, 1, 2), repeat=len(blocks)):
            live = [1 if x else 0 for x in states]
            pin = [1 if x == 2 else 0 for x in states]
            check_against_bruteforce(W.table_from_lists(S, blocks, live, pinned=pin), rng)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**32 - 1), n=st.integers(0, 30),
       gap_p=st.sampled_from([0.0, 0.3, 0.8]), live_p=st.sampled_from([0.0, 0.5, 0.9, 1.0]),
       pinned_p=st.sampled_from([0.0, 0.0, 0.2, 0.5]))
def test_random_tiny_heaps_targeted(seed, n, gap_p, live_p, pinned_p):
    rng = np.random.default_rng(seed)
    heap = W.tiny_heap(rng, n, sizes=(32, 64, 96, 160, 1024), gap_p=gap_p, live_p=live_p,
                       pinned_p=pinned_p)
    check_against_bruteforce(heap, rng)


def check_properties(heap, requests):
    off, size, live, S, pin = heap.offset, heap.size, heap.live, heap.arena_bytes, heap.pinned
    li = np.flatnonzero(live)
    full_new = oracle.new_offsets(off, size, live, pin)
    full = oracle.stats(full_new[li], size[li], np.ones(li.shape[0], np.uint8), S,
                        pinned=None if pin is None else pin[li])
    before = oracle.stats(off, size, live, S, pinned=pin)
    prev_moved = 0
    for R in sorted(requests):
        w = oracle.target_window(off, size, live, S, R, pinned=pin)
        # fits iff a full compaction leaves a hole that large
        assert bool(w.found) == (R <= full.largest_hole), R
        if not w.found:
            continue
        assert w.hole >= R and w.begin < w.end <= S
        assert (w.moved_bytes == 0) == (R <= before.largest_hole)
        assert w.moved_bytes >= prev_moved          # larger request, never cheaper
        prev_moved = w.moved_bytes
        assert w.moved_bytes <= before.moved_bytes  # never more than a full compaction
        fixed = oracle.window_pins(off, live, pin, w)
        plan = oracle.stats(off, size, live, S, pinned=fixed)
        assert plan.moved_bytes == w.moved_bytes
        new = oracle.new_offsets(off, size, live, fixed)
        post = oracle.stats(new[li], size[li], np.ones(li.shape[0], np.uint8), S,
                            pinned=fixed[li])
        assert post.largest_hole >= R
        assert post.free_bytes == before.free_bytes
        # the merged hole sits at the window's top: no live byte in it
        top = w.end - w.hole
        ends = new[li] + size[li]
        assert not np.any((new[li] < w.end) & (ends > top))


@pytest.mark.parametrize("k", ["mixed-64m", "pairs-1g", "training-80g", "small-blocks-4g", "overlap-64g", "training-80g-pinned"])
def test_properties_small_workloads(k, oracle_lib):
    heap = W.workload(k, small=True)
    st_ = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes, pinned=heap.pinned)
    F, L = st_.free_bytes, st_.largest_hole
    reqs = {1, L, L + 1, F // 2, F, F + 1}
    reqs |= {max(1, (F * j) // 16) for j in range(1, 16)}
    check_properties(heap, reqs)


def test_page_request_on_training_80g(oracle_lib):
    """910C page: 14 GB free, largest block under 3 GB, a 4.2 GB buffer
    request fails.  On the workload with those proportions a window that
    frees 4.2/80 of the arena exists and moves a small fraction of what a
    full compaction moves."""
    heap = W.workload("training-80g")
    S = heap.arena_bytes
    R = S * 42 // 800
    before = oracle.stats(heap.offset, heap.size, heap.live, S)
    assert before.largest_hole < R
    w = oracle.target_window(heap.offset, heap.size, heap.live, S, R)
    assert w.found and w.hole >= R
    assert 0 < w.moved_bytes < before.moved_bytes // 4

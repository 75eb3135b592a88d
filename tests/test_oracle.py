"""Pins for the CPU oracle, against things other than the oracle itself.

* hand-worked layouts (tests/golden/hand_worked.json, each case cited);
* a byte-bitmap brute force that states compaction as a stable partition of
  live bytes (tests/bruteforce.py), exhaustively over every live mask of
  small tables and on random tiny heaps;
* the invariants the pages fix: payloads byte-identical at their new place,
  order kept, one top hole afterwards with both ratios 0, free total kept;
* the 910C page's printed ratio on the layout built with its proportions;
* every validation reason, first failing entry wins.
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
U64_MAX = (1 << 64) - 1


def _golden():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)["cases"]


def _table(case):
    t = np.array(case["table"], dtype=np.uint64).reshape(-1, 3)
    pin = np.array(case["pinned"], dtype=np.uint8) if "pinned" in case else None
    return t[:, 0].copy(), t[:, 1].copy(), t[:, 2].astype(np.uint8), pin


def _src_of_each_byte(segments, S):
    src = [None] * S
    for d, s, l in segments:
        for k in range(l):
            assert src[d + k] is None
            src[d + k] = s + k
    return src


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_hand_worked(case, oracle_lib):
    off, size, live, pin = _table(case)
    S = case["arena_bytes"]
    assert oracle.validate(off, size, live, S, pinned=pin)[0] == oracle.OK
    assert oracle.new_offsets(off, size, live, pin).tolist() == case["new_offset"]
    st_ = oracle.stats(off, size, live, S, pinned=pin)
    exp = case["stats"]
    for k in ("arena_bytes", "live_bytes", "free_bytes", "largest_hole", "hole_count",
              "live_blocks", "moved_blocks", "moved_bytes"):
        assert getattr(st_, k) == exp[k], k
    if exp["r1_num_den"] is None:
        assert st_.frag_free_over_largest_minus_1 == 0.0
        assert st_.frag_one_minus_largest_over_free == 0.0
    else:
        n1, d1 = exp["r1_num_den"]
        n2, d2 = exp["r2_num_den"]
        assert st_.frag_free_over_largest_minus_1 == n1 / d1 - 1.0
        assert st_.frag_one_minus_largest_over_free == 1.0 - n2 / d2
    # the moved arena, from the hand-derived source segments
    rng = np.random.default_rng(0)
    A = rng.integers(0, 256, S, dtype=np.uint8)
    B = A.copy()
    oracle.compact(B, off, size, live, pin)
    expect = np.empty_like(A)
    for d, s, l in case["after_move_sources"]:
        expect[d:d + l] = A[s:s + l]
    assert np.array_equal(B, expect)
    d, s, l = oracle.source_map(off, size, live, S, 0, S, pinned=pin)
    assert _src_of_each_byte(zip(d.tolist(), s.tolist(), l.tolist()), S) == \
        _src_of_each_byte(case["after_move_sources"], S)
    h = np.array(case["handles"], dtype=np.uint64)
    out, bad = oracle.remap(off, size, live, h, pinned=pin)
    want = [U64_MAX if v < 0 else v for v in case["remapped"]]
    assert out.tolist() == want
    assert bad == sum(1 for v in case["remapped"] if v < 0)
    if "post_table" in case:
        t = np.array(case["post_table"], dtype=np.uint64)
        ppin = np.array(case["post_pinned"], dtype=np.uint8) if "post_pinned" in case else None
        ps = oracle.stats(t[:, 0], t[:, 1], t[:, 2].astype(np.uint8), S, pinned=ppin)
        pe = case["post_stats"]
        assert (ps.free_bytes, ps.largest_hole, ps.hole_count) == \
            (pe["free_bytes"], pe["largest_hole"], pe["hole_count"])
        assert ps.frag_free_over_largest_minus_1 == pe["r1"]
        assert ps.frag_one_minus_largest_over_free == pe["r2"]


def _check_against_bruteforce(heap):
    off, size, live, S, pin = heap.offset, heap.size, heap.live, heap.arena_bytes, heap.pinned
    assert oracle.validate(off, size, live, S, pinned=pin)[0] == oracle.OK
    # new offsets: segment start + movable live bytes below each entry's start
    assert np.array_equal(oracle.new_offsets(off, size, live, pin),
                          BF.new_offsets(S, off, size, live, pin))
    # arena: stable partition of movable live bytes inside each segment
    rng = np.random.default_rng(int(heap.payload_seed) & 0xFFFF)
    A = rng.integers(0, 256, S, dtype=np.uint8)
    got = A.copy()
    oracle.compact(got, off, size, live, pin)
    assert np.array_equal(got, BF.compacted(A, off, size, live, pin))
    # stats
    exp = BF.stats(S, off, size, live, pin)
    s = oracle.stats(off, size, live, S, pinned=pin)
    for k, v in exp.items():
        assert getattr(s, k) == v, (k, getattr(s, k), v)
    # remap: rank of the byte among movable live bytes of its segment
    out, bad = oracle.remap(off, size, live, heap.handles, pinned=pin)
    eo, eb = BF.remap(S, off, size, live, heap.handles, pin)
    assert np.array_equal(out, eo) and bad == eb
    # the source map rebuilds the same compacted arena
    d, s_, l = oracle.source_map(off, size, live, S, 0, S, pinned=pin)
    rebuilt = np.empty_like(A)
    for dd, ss, ll in zip(d.tolist(), s_.tolist(), l.tolist()):
        rebuilt[dd:dd + ll] = A[ss:ss + ll]
    assert np.array_equal(rebuilt, got)


def test_exhaustive_live_masks(oracle_lib):
    """Every live mask over fixed tables of up to 8 entries, with and
    without untracked gaps and tail."""
    layouts = [
        [(0, 32), (32, 64), (96, 96), (192, 32), (224, 64), (288, 32), (320, 96), (416, 32)],
        [(32, 32), (96, 64), (160, 96), (288, 32), (320, 32), (384, 64), (512, 32), (576, 96)],
    ]
    for blocks in layouts:
        for n in range(0, len(blocks) + 1):
            bl = blocks[:n]
            end = bl[-1][0] + bl[-1][1] if bl else 0
            for tail in (0, 64):
                S = end + tail
                for mask in itertools.product((0, 1), repeat=n):
                    h = W.table_from_lists(S, bl, mask)
                    rng = np.random.default_rng(n * 1000 + sum(mask))
                    h.handles = W.edge_handles(h, rng, 4)
                    _check_against_bruteforce(h)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**32 - 1), n=st.integers(0, 40),
       gap_p=st.sampled_from([0.0, 0.3, 0.8]), live_p=st.sampled_from([0.0, 0.5, 0.9, 1.0]),
       pinned_p=st.sampled_from([0.0, 0.0, 0.2, 0.5]))
def test_random_tiny_heaps(seed, n, gap_p, live_p, pinned_p):
    rng = np.random.default_rng(seed)
    heap = W.tiny_heap(rng, n, sizes=(32, 64, 96, 160, 4096), gap_p=gap_p, live_p=live_p,
                       pinned_p=pinned_p)
    _check_against_bruteforce(heap)


def test_exhaustive_pinned_masks(oracle_lib):
    """Every (free, live, pinned) assignment over a 5-entry table with gaps."""
    blocks = [(32, 32), (64, 64), (160, 96), (256, 32), (320, 64)]
    for tail in (0, 96):
        S = 384 + tail
        for states in itertools.product((0, 1, 2), repeat=len(blocks)):
            live = [1 if x else 0 for x in states]
            pin = [1 if x == 2 else 0 for x in states]
            h = W.table_from_lists(S, blocks, live, pinned=pin)
            h.handles = W.edge_handles(h, np.random.default_rng(sum(states)), 4)
            _check_against_bruteforce(h)


@pytest.mark.parametrize("k", ["mixed-64m", "pairs-1g", "training-80g", "small-blocks-4g", "overlap-64g"])
def test_invariants_small_workloads(k, oracle_lib):
    """I1-I6 on the reduced workloads, with the real payload generator."""
    import torch
    heap = W.workload(k, small=True)
    off, size, live, S = heap.offset, heap.size, heap.live, heap.arena_bytes
    assert oracle.validate(off, size, live, S)[0] == oracle.OK
    new = oracle.new_offsets(off, size, live)
    li = np.flatnonzero(live)
    # I1/I2: first live block lands at 0, the next starts where the last ends
    if li.shape[0]:
        assert new[li[0]] == 0
        assert np.array_equal(new[li[1:]], new[li[:-1]] + size[li[:-1]])
    lt = int(size[li].sum())
    A = torch.empty(S, dtype=torch.uint8)
    W.fill_payload(A, 0, heap.payload_mode, heap.payload_seed)
    A = A.numpy()
    got = A.copy()
    oracle.compact(got, off, size, live)
    # I3: every live payload byte-identical at its new place (order kept)
    for i in li.tolist()[:: max(1, li.shape[0] // 2000)] + li.tolist()[-3:]:
        o, s, nw = int(off[i]), int(size[i]), int(new[i])
        assert np.array_equal(got[nw:nw + s], A[o:o + s]), i
    # I4: bytes at or above the live total untouched
    assert np.array_equal(got[lt:], A[lt:])
    before = oracle.stats(off, size, live, S)
    # I5/I6: after compaction one top hole, both ratios 0, same free total
    pt = oracle.stats(new[li], size[li], np.ones(li.shape[0], np.uint8), S)
    assert pt.free_bytes == before.free_bytes == S - lt
    assert pt.hole_count == (1 if S > lt else 0)
    assert pt.largest_hole == S - lt
    assert pt.frag_free_over_largest_minus_1 == 0.0
    assert pt.frag_one_minus_largest_over_free == 0.0
    assert pt.moved_blocks == 0
    # remap: closed form h - shift for in-block handles, end to end on bytes
    out, bad = oracle.remap(off, size, live, heap.handles)
    assert bad == 0   # the workload's handles all sit inside live blocks
    hs = heap.handles[:5000]
    assert np.array_equal(got[out[:5000].astype(np.int64)], A[hs.astype(np.int64)])


def test_training_80g_page_proportions(oracle_lib):
    """910C page, monitoring section: the ratio free/largest - 1 reached 4.7
    with 14 GB free; the workload built with those proportions must read 4.7
    (and 1 - largest/free = 1 - 1/5.7 = 0.8246) through the oracle."""
    heap = W.workload("training-80g")
    s = oracle.stats(heap.offset, heap.size, heap.live, heap.arena_bytes)
    assert s.free_bytes == 14 * W.GiB
    assert s.largest_hole == heap.notes["largest_target"] == 2_637_258_752
    assert abs(s.frag_free_over_largest_minus_1 - 4.7) < 1e-3
    assert abs(s.frag_one_minus_largest_over_free - (1 - 1 / 5.7)) < 1e-4
    assert s.live_bytes == 66 * W.GiB
    # after compaction both ratios are 0 (CANN page 3.3: one free region)
    li = np.flatnonzero(heap.live)
    new = oracle.new_offsets(heap.offset, heap.size, heap.live)
    pt = oracle.stats(new[li], heap.size[li], np.ones(li.shape[0], np.uint8), heap.arena_bytes)
    assert pt.hole_count == 1 and pt.largest_hole == 14 * W.GiB
    assert pt.frag_free_over_largest_minus_1 == 0.0 == pt.frag_one_minus_largest_over_free


@pytest.mark.parametrize("table,S,idx,reason", [
    ([(0, 0, 1)], 64, 0, 1),
    ([(0, 32, 1), (32, 0, 0)], 64, 1, 1),
    ([(16, 32, 1)], 64, 0, 2),
    ([(0, 48, 1)], 64, 0, 2),
    ([(0, 32, 2)], 64, 0, 3),
    ([(0, 32, 1), (32, 64, 1)], 64, 1, 4),
    ([(96, 32, 1)], 64, 0, 4),
    ([(0, 64, 1), (32, 32, 0)], 128, 1, 5),
    ([(64, 32, 1), (0, 32, 1)], 128, 1, 5),
    ([(0, 32, 1), (0, 32, 1)], 128, 1, 5),
    ([(0, 32, 1), (64, 32, 0), (64, 0, 1)], 128, 2, 1),
    ([(0, 32, 1), (1 << 63, 1 << 63, 1)], 1 << 63, 1, 4),
    ([(2**64 - 48, 32, 1)], U64_MAX, 0, 2),
    ([(2**64 - 32, 32, 1)], U64_MAX, 0, 4),
    ([(2**64 - 64, 64, 1)], U64_MAX, 0, 4),
])
def test_validation_reasons(table, S, idx, reason, oracle_lib):
    t = np.array(table, dtype=np.uint64)
    rc, bad, r = oracle.validate(t[:, 0], t[:, 1], t[:, 2].astype(np.uint8), S)
    assert (rc, bad, r) == (oracle.EINVAL, idx, reason)


def test_empty_and_degenerate(oracle_lib):
    e = np.zeros(0, np.uint64)
    el = np.zeros(0, np.uint8)
    assert oracle.validate(e, e, el, 0)[0] == oracle.OK
    s = oracle.stats(e, e, el, 0)
    assert (s.free_bytes, s.largest_hole, s.hole_count) == (0, 0, 0)
    assert s.frag_free_over_largest_minus_1 == 0.0
    s = oracle.stats(e, e, el, 4096)
    assert (s.free_bytes, s.largest_hole, s.hole_count) == (4096, 4096, 1)
    assert s.frag_free_over_largest_minus_1 == 0.0 and s.frag_one_minus_largest_over_free == 0.0
    out, bad = oracle.remap(e, e, el, np.array([0, 5], np.uint64))
    assert bad == 2 and out.tolist() == [U64_MAX, U64_MAX]
    d, s_, l = oracle.source_map(e, e, el, 4096, 100, 50)
    assert (d.tolist(), s_.tolist(), l.tolist()) == ([100], [100], [50])


def _check_source_map_windows(heap, rng, n_windows=12):
    """Any window of the source map equals that slice of the compacted arena
    (windows start and end inside blocks, holes and the tail)."""
    S = heap.arena_bytes
    A = rng.integers(0, 256, S, dtype=np.uint8)
    got = A.copy()
    oracle.compact(got, heap.offset, heap.size, heap.live, heap.pinned)
    for _ in range(n_windows):
        if S == 0:
            break
        p0 = int(rng.integers(0, S))
        ln = int(rng.integers(1, S - p0 + 1))
        d, s, l = oracle.source_map(heap.offset, heap.size, heap.live, S, p0, ln,
                                    pinned=heap.pinned)
        rebuilt = np.full(ln, -1, dtype=np.int16)
        for dd, ss, ll in zip(d.tolist(), s.tolist(), l.tolist()):
            rebuilt[dd - p0:dd - p0 + ll] = A[ss:ss + ll]
        assert np.array_equal(rebuilt, got[p0:p0 + ln].astype(np.int16)), (p0, ln)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**32 - 1), n=st.integers(1, 30))
def test_source_map_any_window(seed, n):
    rng = np.random.default_rng(seed)
    heap = W.tiny_heap(rng, n, sizes=(32, 64, 96, 160), gap_p=0.4, live_p=0.6,
                       pinned_p=0.25 if seed % 2 else 0.0)
    _check_source_map_windows(heap, rng)


@pytest.mark.parametrize("table,pinned,S,idx,reason", [
    ([(0, 32, 1)], [2], 64, 0, 7),
    ([(0, 32, 0)], [1], 64, 0, 7),
    ([(0, 32, 1), (32, 32, 0)], [0, 1], 64, 1, 7),
    ([(0, 32, 2)], [1], 64, 0, 3),            # live flag is checked before pinned
    ([(0, 32, 0), (96, 32, 1)], [1, 0], 64, 0, 7),   # pinned before out of arena
    ([(0, 32, 1), (96, 32, 1)], [1, 1], 64, 1, 4),
    ([(0, 64, 1), (32, 32, 1)], [1, 1], 128, 1, 5),
])
def test_validation_reasons_pinned(table, pinned, S, idx, reason, oracle_lib):
    t = np.array(table, dtype=np.uint64)
    rc, bad, r = oracle.validate(t[:, 0], t[:, 1], t[:, 2].astype(np.uint8), S,
                                 pinned=np.array(pinned, np.uint8))
    assert (rc, bad, r) == (oracle.EINVAL, idx, reason)


def test_pinned_segments_invariants(oracle_lib):
    """Reduced training-80g with its 40 parameter/optimizer blocks pinned: pinned
    bytes never change; every segment's movable blocks are packed from the
    segment start in order, payload intact; afterwards every segment holds at
    most one hole, at its top, and the free total is unchanged."""
    import torch
    heap = W.workload("training-80g-pinned", small=True)
    off, size, live, pin, S = heap.offset, heap.size, heap.live, heap.pinned, heap.arena_bytes
    assert heap.n_pinned == 40
    assert oracle.validate(off, size, live, S, pinned=pin)[0] == oracle.OK
    new = oracle.new_offsets(off, size, live, pin)
    A = torch.empty(S, dtype=torch.uint8)
    W.fill_payload(A, 0, heap.payload_mode, heap.payload_seed)
    A = A.numpy()
    got = A.copy()
    oracle.compact(got, off, size, live, pin)
    seg_start = 0
    cursor = 0
    for i in range(heap.n):
        o, s_ = int(off[i]), int(size[i])
        if pin[i]:
            assert int(new[i]) == o and np.array_equal(got[o:o + s_], A[o:o + s_])
            seg_start = cursor = o + s_
            continue
        if live[i]:
            assert int(new[i]) == cursor >= seg_start
            if i % 97 == 0 or s_ > (1 << 20):
                assert np.array_equal(got[cursor:cursor + s_], A[o:o + s_]), i
            cursor += s_
    li = np.flatnonzero(live)
    before = oracle.stats(off, size, live, S, pinned=pin)
    pt = oracle.stats(new[li], size[li], np.ones(li.shape[0], np.uint8), S, pinned=pin[li])
    assert pt.free_bytes == before.free_bytes
    assert pt.moved_blocks == 0
    # at most one hole per segment: segments = pinned blocks + 1
    assert pt.hole_count <= heap.n_pinned + 1
    assert pt.largest_hole < before.free_bytes   # the pinned blocks keep free space apart
    out, bad = oracle.remap(off, size, live, heap.handles, pinned=pin)
    assert bad == 0
    assert np.array_equal(got[out[:5000].astype(np.int64)], A[heap.handles[:5000].astype(np.int64)])

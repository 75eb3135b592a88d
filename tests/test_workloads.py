"""The seeded input generators: payload function and workload shapes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def test_splitmix64_published_outputs():
    """First outputs of SplitMix64 seeded with 1234567, as published with the
    reference C implementation (splitmix64.c, Vigna)."""
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [W.splitmix64_py(1234567, k) for k in range(5)] == want
    t = torch.empty(40, dtype=torch.uint8)
    W.fill_payload(t, 0, "hash", 1234567)
    got = [int(v) & W.U64_MAX for v in t.view(torch.int64).tolist()]
    assert got == want


@pytest.mark.parametrize("seed", [0, 7, 0xC0FFEE03, (1 << 64) - 1])
def test_hash_payload_random_access(seed):
    rng = np.random.default_rng(1)
    for w in rng.integers(0, 1 << 40, 20).tolist() + [0, 1, (1 << 40) - 1]:
        a = w * 8
        t = torch.empty(16, dtype=torch.uint8)
        W.fill_payload(t, a, "hash", seed)
        got = [int(v) & W.U64_MAX for v in t.view(torch.int64).tolist()]
        assert got == [W.splitmix64_py(seed, w), W.splitmix64_py(seed, w + 1)]
    # unaligned windows are slices of the aligned stream
    big = W.payload_window(4096, 256, "hash", seed)
    for a, l in [(4097, 5), (4100, 100), (4352 - 3, 3)]:
        assert np.array_equal(W.payload_window(a, l, "hash", seed), big[a - 4096:a - 4096 + l])


def test_counter32_payload():
    seed = 0x5EED0005
    t = torch.empty(64, dtype=torch.uint8)
    base = (1 << 34) + 64  # word index past 2**32: wraps modulo 2**32
    W.fill_payload(t, base, "counter32", seed)
    words = t.numpy().view(np.uint32)
    j = np.arange(base // 4, base // 4 + 16, dtype=np.uint64)
    assert np.array_equal(words, ((j & np.uint64(0xFFFFFFFF)) ^ np.uint64(seed)).astype(np.uint32))


def test_chunked_fill_matches_single():
    a = torch.empty(1 << 16, dtype=torch.uint8)
    b = torch.empty(1 << 16, dtype=torch.uint8)
    W.fill_payload(a, 8192, "hash", 3)
    W.fill_payload(b, 8192, "hash", 3, chunk_bytes=1000)
    assert torch.equal(a, b)


def _valid(heap):
    rc, bad, r = oracle.validate(heap.offset, heap.size, heap.live, heap.arena_bytes)
    assert rc == oracle.OK, (bad, r)


def _handles_inside_live(heap):
    h = heap.handles
    i = np.searchsorted(heap.offset, h, side="right") - 1
    assert np.all(i >= 0)
    assert np.all(heap.live[i] == 1)
    assert np.all(h - heap.offset[i] < heap.size[i])


def test_mixed_64m_shape():
    h = W.workload("mixed-64m")
    _valid(h)
    assert h.n == 4096 and h.arena_bytes == 64 * W.MiB
    assert np.all(h.size % 32 == 0) and h.size.min() >= 256 and h.size.max() <= 64 * W.KiB
    assert np.array_equal(h.offset[1:], h.offset[:-1] + h.size[:-1])   # packed
    assert abs(h.live.mean() - 0.5) < 0.05
    assert h.handles.shape[0] == 16384
    _handles_inside_live(h)


def test_pairs_1g_shape():
    h = W.workload("pairs-1g")
    _valid(h)
    assert h.n == 65536 and h.arena_bytes == W.GiB
    assert np.all(h.size % 512 == 0)
    assert np.array_equal(h.size[1::2], 2 * h.size[0::2])
    assert abs(h.live.mean() - 0.6) < 0.02
    assert h.handles.shape[0] == 1_000_000
    _handles_inside_live(h)


def test_training_80g_shape():
    h = W.workload("training-80g")
    _valid(h)
    assert h.arena_bytes == 80 * W.GiB
    assert np.all(h.size % 4096 == 0)
    assert int((h.size * h.live).sum()) == 66 * W.GiB
    assert int(h.offset[-1] + h.size[-1]) == h.arena_bytes   # no untracked tail
    assert h.handles.shape[0] == 4_000_000
    # no two free entries adjacent (each freed block is its own hole)
    fl = h.live == 0
    assert not np.any(fl[1:] & fl[:-1])
    _handles_inside_live(h)


def test_small_blocks_4g_shape():
    h = W.workload("small-blocks-4g")
    _valid(h)
    assert h.n == 2_000_000 and h.arena_bytes == 4 * W.GiB
    assert np.all(h.size % 32 == 0) and h.size.min() >= 32 and h.size.max() <= 4096
    assert h.live[0] == 0 and np.all(h.live[1::2] == 1) and np.all(h.live[0::2] == 0)
    assert h.handles.shape[0] == 8_000_000
    _handles_inside_live(h)


def test_overlap_64g_shape():
    h = W.workload("overlap-64g")
    _valid(h)
    assert h.n == 128
    assert np.all(h.size[1::2] == W.GiB) and np.all(h.live[1::2] == 1)
    holes = h.size[0::2]
    assert holes.min() >= 4 * W.KiB and holes.max() <= 64 * W.MiB and np.all(holes % 32 == 0)
    assert h.arena_bytes == 64 * W.GiB + int(holes.sum())
    assert h.payload_mode == "counter32"
    _handles_inside_live(h)


def test_small_shift_8g_shape():
    h = W.workload("small-shift-8g")
    _valid(h)
    assert h.n == 16
    assert np.all(h.size[1::2] == W.GiB) and np.all(h.live[1::2] == 1) and np.all(h.live[0::2] == 0)
    holes = h.size[0::2]
    assert holes.min() >= 4 * W.KiB and holes.max() <= W.MiB and np.all(holes % 32 == 0)
    assert h.arena_bytes == 8 * W.GiB + int(holes.sum())
    assert h.handles.shape[0] == 1_000_000
    _handles_inside_live(h)


@pytest.mark.parametrize("k", W.NAMES)
def test_small_variants_valid_and_seeded(k):
    a = W.workload(k, small=True)
    b = W.workload(k, small=True)
    _valid(a)
    assert np.array_equal(a.offset, b.offset) and np.array_equal(a.live, b.live)
    assert np.array_equal(a.handles, b.handles)

"""Seeded synthetic heaps for the arena compactor.

This module only *draws inputs*: block tables (offset, size, live flag),
handles, and the pristine arena payload.  It holds none of the compactor's
arithmetic (no live-size scan, no hole statistics, no moves, no remap); both
the HIP path and the CPU oracle consume what it produces.

The five workloads follow the heap shapes of the Ascend 910C fragmentation
page ("Ascend 910C cluster tuning: memory-fragment compaction in
mixed-precision training") and the CANN memory page ("CANN memory
management and optimisation"): 32-byte granularity (CANN page, section 2.2
memory pool, 32 B rounding; section 3.3 aligned allocation), a mix of large
long-lived parameter/optimizer blocks, mid-sized activations and many small
tensors, with freed holes between them (910C page, section on why 14 GB of
free HBM could not be used).

Units: KiB/MiB/GiB are binary; "k"/"M" counts are decimal (2M = 2,000,000).
Sizes drawn from a continuous law are rounded *up* to the granularity, as the
CANN pool rounds every request up to 32 bytes.

Payload: the pristine arena content is a pure function of the byte address,
so any window can be recomputed anywhere (CPU or GPU) without storing it.
  * ``hash``  : 8-byte word w = output number w of a SplitMix64 stream seeded
                with ``seed`` (Steele, Lea & Flood, "Fast splittable
                pseudorandom number generators", OOPSLA 2014; constants as in
                Vigna's public-domain splitmix64.c), little-endian.
  * ``counter32`` : 4-byte word j = (j mod 2**32) XOR seed.
The same torch code fills CPU tensors (oracle side) and HIP tensors (device
side), so both sides start from identical bytes by construction.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional

import numpy as np
import torch

KiB = 1 << 10
MiB = 1 << 20
GiB = 1 << 30
U64_MAX = (1 << 64) - 1

# SplitMix64 constants (golden-ratio increment and the two mixing multipliers).
_SM_GAMMA = 0x9E3779B97F4A7C15
_SM_M1 = 0xBF58476D1CE4E5B9
_SM_M2 = 0x94D049BB133111EB


def _s64(x: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64 (same bits)."""
    x &= U64_MAX
    return x - (1 << 64) if x >= (1 << 63) else x


def splitmix64_py(seed: int, k: int) -> int:
    """Output number ``k`` (0-based) of a SplitMix64 stream seeded with
    ``seed``: state advances by the golden gamma before every output, then
    the 64-bit finaliser is applied.  Pure-Python reference for tests."""
    z = (seed + (k + 1) * _SM_GAMMA) & U64_MAX
    z = ((z ^ (z >> 30)) * _SM_M1) & U64_MAX
    z = ((z ^ (z >> 27)) * _SM_M2) & U64_MAX
    return z ^ (z >> 31)


def _splitmix64_words_(z: torch.Tensor, seed: int) -> torch.Tensor:
    """In place: z holds word indices k (int64); returns SplitMix64 output k.

    int64 multiply wraps modulo 2**64 (two's complement), which is the
    unsigned arithmetic SplitMix64 needs; right shifts are made logical by
    masking the sign-extended high bits.
    """
    z.add_(1).mul_(_s64(_SM_GAMMA)).add_(_s64(seed))
    t = torch.bitwise_right_shift(z, 30).bitwise_and_((1 << 34) - 1)
    z.bitwise_xor_(t).mul_(_s64(_SM_M1))
    torch.bitwise_right_shift(z, 27, out=t).bitwise_and_((1 << 37) - 1)
    z.bitwise_xor_(t).mul_(_s64(_SM_M2))
    torch.bitwise_right_shift(z, 31, out=t).bitwise_and_((1 << 33) - 1)
    z.bitwise_xor_(t)
    return z


_HERE = os.path.dirname(os.path.abspath(__file__))
_CLIB_PATH = os.path.join(_HERE, "libworkloads.so")
_clib = None


def build_host_generator(verbose: bool = False) -> str:
    """Compile the C payload generator used for CPU buffers."""
    cmd = ["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o",
           _CLIB_PATH + ".tmp", os.path.join(_HERE, "payload.c")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_CLIB_PATH + ".tmp", _CLIB_PATH)
    return _CLIB_PATH


def _host_lib():
    global _clib
    if _clib is None:
        src = os.path.join(_HERE, "payload.c")
        if not os.path.exists(_CLIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_CLIB_PATH):
            build_host_generator()
        L = ctypes.CDLL(_CLIB_PATH)
        L.wl_fill_hash.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_uint64]
        L.wl_fill_counter32.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_uint32]
        _clib = L
    return _clib


def fill_payload(dst: torch.Tensor, base_addr: int, mode: str, seed: int,
                 chunk_bytes: int = 256 * MiB, use_torch: bool = False) -> None:
    """Write the pristine payload of arena bytes [base_addr, base_addr+len)
    into the 1-D uint8 tensor ``dst`` (CPU or GPU).

    ``base_addr`` and ``len(dst)`` must be multiples of 8 (hash) or 4
    (counter32).  GPU tensors are filled with torch ops in bounded chunks;
    CPU tensors with the equivalent C loop (``use_torch`` forces the torch
    code on the CPU too, to pin the two against each other).
    """
    assert dst.dtype == torch.uint8 and dst.dim() == 1 and dst.is_contiguous()
    n = dst.numel()
    if mode == "hash":
        wb = 8
    elif mode == "counter32":
        wb = 4
    else:
        raise ValueError(f"unknown payload mode {mode!r}")
    if base_addr % wb or n % wb:
        raise ValueError("payload window must be word aligned")
    if n == 0:
        return
    if not dst.is_cuda and not use_torch:
        L = _host_lib()
        if mode == "hash":
            L.wl_fill_hash(dst.data_ptr(), base_addr // 8, n // 8, seed & U64_MAX)
        else:
            L.wl_fill_counter32(dst.data_ptr(), base_addr // 4, n // 4, seed & 0xFFFFFFFF)
        return
    dev = dst.device
    step = max(wb, (chunk_bytes // wb) * wb)
    for c0 in range(0, n, step):
        c1 = min(n, c0 + step)
        cnt = (c1 - c0) // wb
        w0 = (base_addr + c0) // wb
        z = torch.arange(w0, w0 + cnt, dtype=torch.int64, device=dev)
        if mode == "hash":
            _splitmix64_words_(z, seed)
            dst[c0:c1].view(torch.int64).copy_(z)
        else:
            z.bitwise_and_(0xFFFFFFFF).bitwise_xor_(seed & 0xFFFFFFFF)
            # values are in [0, 2**32): keep the low 32 bits, two's complement
            z = torch.where(z >= (1 << 31), z - (1 << 32), z)
            dst[c0:c1].view(torch.int32).copy_(z.to(torch.int32))
        del z


def payload_window(base_addr: int, length: int, mode: str, seed: int) -> np.ndarray:
    """Pristine bytes of [base_addr, base_addr+length) as a numpy uint8 array
    (computed on the CPU; handles unaligned windows)."""
    wb = 8 if mode == "hash" else 4
    a0 = (base_addr // wb) * wb
    a1 = ((base_addr + length + wb - 1) // wb) * wb
    t = torch.empty(a1 - a0, dtype=torch.uint8)
    fill_payload(t, a0, mode, seed)
    off = base_addr - a0
    return t.numpy()[off:off + length].copy()


@dataclasses.dataclass
class Heap:
    """A block table over an arena of ``arena_bytes`` bytes.

    offset/size are uint64, live is uint8 (0/1); entries ascending and
    non-overlapping for every generated heap (tests that need invalid tables
    build them by hand).  ``handles`` are byte addresses (uint64).
    """
    name: str
    arena_bytes: int
    offset: np.ndarray
    size: np.ndarray
    live: np.ndarray
    handles: np.ndarray
    payload_mode: str = "hash"
    payload_seed: int = 0
    seed: int = 0
    notes: dict = dataclasses.field(default_factory=dict)
    pinned: Optional[np.ndarray] = None   # uint8 0/1 per entry, or None: nothing pinned

    @property
    def n(self) -> int:
        return int(self.offset.shape[0])

    @property
    def n_pinned(self) -> int:
        return 0 if self.pinned is None else int(self.pinned.sum())

    def describe(self) -> str:
        return (f"{self.name}: S={self.arena_bytes} n={self.n} "
                f"live={int(self.live.sum())} pinned={self.n_pinned} "
                f"handles={self.handles.shape[0]} seed={self.seed}")


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def _ceil_to(x: np.ndarray, g: int) -> np.ndarray:
    x = np.asarray(x)
    return ((np.ceil(x / g)).astype(np.uint64)) * np.uint64(g)


def _loguniform(rng: np.random.Generator, lo: float, hi: float, k: int) -> np.ndarray:
    return np.exp(rng.uniform(math.log(lo), math.log(hi), k))


def _packed_offsets(sizes: np.ndarray, base: int = 0) -> np.ndarray:
    """Back-to-back layout: block k starts where block k-1 ends (all blocks,
    live or not -- this is how the heap was allocated, not the compaction)."""
    off = np.empty_like(sizes)
    if sizes.shape[0]:
        off[0] = base
        np.cumsum(sizes[:-1], out=off[1:])
        off[1:] += np.uint64(base)
    return off


def draw_handles(offset: np.ndarray, size: np.ndarray, live: np.ndarray,
                 count: int, rng: np.random.Generator) -> np.ndarray:
    """``count`` handles at uniformly random byte positions inside uniformly
    chosen live blocks (a live block first, then an offset in it)."""
    live_idx = np.flatnonzero(live)
    if count == 0 or live_idx.shape[0] == 0:
        return np.zeros(0, dtype=np.uint64)
    pick = live_idx[rng.integers(0, live_idx.shape[0], count)]
    frac = rng.random(count)
    inner = np.floor(frac * size[pick].astype(np.float64)).astype(np.uint64)
    inner = np.minimum(inner, size[pick] - np.uint64(1))
    return offset[pick] + inner


def edge_handles(heap: Heap, rng: np.random.Generator, extra_random: int = 64) -> np.ndarray:
    """Handles that probe the edges: every block's first and last byte, one
    past every block's end, the arena end and beyond, 0, and some uniform
    addresses over the whole arena (many of which fall in holes)."""
    off, size = heap.offset, heap.size
    parts = [off, off + size - np.uint64(1), off + size,
             np.array([0, heap.arena_bytes, heap.arena_bytes + 1,
                       max(heap.arena_bytes, 1) - 1, U64_MAX, U64_MAX - 31],
                      dtype=np.uint64)]
    if heap.arena_bytes > 0 and extra_random:
        parts.append(rng.integers(0, heap.arena_bytes, extra_random,
                                  dtype=np.uint64))
    return np.concatenate(parts).astype(np.uint64)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def mixed_64mib(seed: int = 1, n_blocks: int = 4096, arena_bytes: int = 64 * MiB,
            n_handles: int = 16384) -> Heap:
    """64 MiB arena, 4,096 blocks of log-uniform 256 B..64 KiB (ceil to 32 B),
    packed from 0, untracked free tail; each block live with p = 0.5."""
    rng = np.random.default_rng(seed)
    size = _ceil_to(_loguniform(rng, 256, 64 * KiB, n_blocks), 32)
    off = _packed_offsets(size)
    assert int(off[-1] + size[-1]) <= arena_bytes
    live = (rng.random(n_blocks) < 0.5).astype(np.uint8)
    h = draw_handles(off, size, live, n_handles, rng)
    return Heap("mixed-64m", arena_bytes, off, size, live, h, "hash",
                0xC0FFEE00 + seed, seed)


def pairs_1gib(seed: int = 2, n_pairs: int = 32768, arena_bytes: int = 1 * GiB,
            n_handles: int = 1_000_000) -> Heap:
    """1 GiB arena, 65,536 blocks as 32,768 interleaved pairs (b, 2b) -- a
    BF16-like tensor followed by an FP32-like one -- with b a multiple of
    512 B.  b is log-uniform 4 KiB..1 MiB divided by 32, ceil to 512 B: at
    the undivided sizes a pair averages about 0.54 MiB and 32,768 pairs
    would need some 17 GiB, so the law is scaled to fill about half of the
    1 GiB arena.  Live p = 0.6."""
    rng = np.random.default_rng(seed)
    b = _ceil_to(_loguniform(rng, 4 * KiB, 1 * MiB, n_pairs) / 32.0, 512)
    size = np.empty(2 * n_pairs, dtype=np.uint64)
    size[0::2] = b
    size[1::2] = b * np.uint64(2)
    off = _packed_offsets(size)
    assert int(off[-1] + size[-1]) <= arena_bytes
    live = (rng.random(2 * n_pairs) < 0.6).astype(np.uint8)
    h = draw_handles(off, size, live, n_handles, rng)
    return Heap("pairs-1g", arena_bytes, off, size, live, h, "hash",
                0xC0FFEE00 + seed, seed)


def training_80gib(seed: int = 3, arena_bytes: int = 80 * GiB, n_pinned: int = 40,
            n_act: int = 200, n_small: int = 200_000, gran: int = 4 * KiB,
            n_handles: int = 4_000_000, pin_params: bool = False) -> Heap:
    """An arena shaped like the 910C page's failure: 14/80 of the arena free,
    largest hole = floor_g(free / 5.7) so that free/largest - 1 = 4.7.

    Low to high: 20 pinned parameter blocks | the freed 4.2/80-of-arena
    communication gap, re-cut by one small live block | 20 pinned optimizer
    blocks | a shuffled mix of activation and small blocks with four named
    holes (two of the largest size, two of 1/80 of the arena) at seeded
    positions.  All block populations are scaled by one factor so the layout
    tiles the arena exactly; random non-adjacent activation/small blocks are
    then freed until the free total is exactly 14/80 of the arena.
    Sizes are multiples of ``gran``.

    With ``pin_params`` the 40 parameter/optimizer blocks are pinned (fixed
    addresses, as the 910C page's parameter region in "cutting alloc and free
    at the source"): the same table, but those blocks may not move.
    """
    rng = np.random.default_rng(seed)
    S = arena_bytes
    g = gran

    def floor_g(x: int) -> int:
        return (x // g) * g

    F = S * 14 // 80                      # free total ("14 GB of 96" shape)
    assert F % g == 0
    L = floor_g(F * 10 // 57)             # largest hole: F / 5.7
    one = floor_g(S // 80)                # "1 GiB" at the 80 GiB scale
    G = floor_g(S * 42 // 800)            # the 4.2 GiB comm-buffer gap
    half = floor_g((G - g) // 2)
    named_free = 2 * L + 2 * one + 2 * half
    assert half <= L and one <= L

    # --- draw the three populations, then scale them to tile the arena ---
    pinned = rng.uniform(1.0, 2.0, n_pinned) * GiB
    act = _loguniform(rng, 8 * MiB, 512 * MiB, n_act)
    small = _loguniform(rng, 4 * KiB, 1 * MiB, n_small)
    target = S - named_free - g           # minus the block splitting the gap
    alpha = target / float(pinned.sum() + act.sum() + small.sum())
    pin_sz = _ceil_to(pinned * alpha, g)
    act_sz = _ceil_to(act * alpha, g)
    small_sz = _ceil_to(small * alpha, g)
    resid = target - int(pin_sz.sum() + act_sz.sum() + small_sz.sum())
    pin_sz[-1] = np.uint64(int(pin_sz[-1]) + resid)   # rounding residual
    assert int(pin_sz[-1]) > 0

    # kinds: 0 pinned, 1 activation, 2 small, 3 named hole, 4 gap half, 5 gap splitter
    mixed_sz = np.concatenate([act_sz, small_sz])
    mixed_kind = np.concatenate([np.full(n_act, 1, np.uint8),
                                 np.full(n_small, 2, np.uint8)])
    perm = rng.permutation(mixed_sz.shape[0])
    mixed_sz, mixed_kind = mixed_sz[perm], mixed_kind[perm]
    # four named holes at distinct, non-adjacent seeded positions
    nm = mixed_sz.shape[0]
    while True:
        pos = np.sort(rng.choice(np.arange(1, nm), 4, replace=False))
        if np.all(np.diff(pos) > 1):
            break
    hole_sizes = np.array([L, L, one, one], dtype=np.uint64)[rng.permutation(4)]
    mixed_sz = np.insert(mixed_sz, pos, hole_sizes)
    mixed_kind = np.insert(mixed_kind, pos, np.full(4, 3, np.uint8))

    half_p = n_pinned // 2
    size = np.concatenate([
        pin_sz[:half_p],
        np.array([half, g, half], dtype=np.uint64),
        pin_sz[half_p:],
        mixed_sz]).astype(np.uint64)
    kind = np.concatenate([
        np.zeros(half_p, np.uint8), np.array([4, 5, 4], np.uint8),
        np.zeros(n_pinned - half_p, np.uint8), mixed_kind])
    live = np.isin(kind, (0, 1, 2, 5)).astype(np.uint8)
    off = _packed_offsets(size)
    assert int(off[-1] + size[-1]) == S

    # --- free random activation/small blocks (not next to a free entry) ---
    remaining = F - named_free
    cand = np.flatnonzero(np.isin(kind, (1, 2)))
    cand = cand[rng.permutation(cand.shape[0])]
    n = size.shape[0]
    for i in cand:
        if remaining == 0:
            break
        s = int(size[i])
        if s > remaining:
            continue
        if (i > 0 and live[i - 1] == 0) or (i + 1 < n and live[i + 1] == 0):
            continue
        live[i] = 0
        remaining -= s
    assert remaining == 0, "could not reach the free-total target exactly"

    h = draw_handles(off, size, live, n_handles, rng)
    heap = Heap("training-80g" + ("-pinned" if pin_params else ""), S, off, size, live, h, "hash",
                0xC0FFEE00 + seed, seed)
    heap.notes.update(dict(free_target=F, largest_target=L, alpha=alpha,
                           named_free=named_free, gap=2 * half + g))
    if pin_params:
        heap.pinned = (kind == 0).astype(np.uint8)
    return heap


def small_blocks_4gib(seed: int = 4, n_blocks: int = 2_000_000, arena_bytes: int = 4 * GiB,
            n_handles: int = 8_000_000) -> Heap:
    """Adversarial small-block heap: 2,000,000 blocks of 32 * U{1..128} bytes,
    packed; block 0 free, then strictly alternating live/free so every live
    block moves; free tail."""
    rng = np.random.default_rng(seed)
    size = (rng.integers(1, 129, n_blocks).astype(np.uint64) * np.uint64(32))
    off = _packed_offsets(size)
    assert int(off[-1] + size[-1]) <= arena_bytes
    live = (np.arange(n_blocks) % 2 == 1).astype(np.uint8)
    h = draw_handles(off, size, live, n_handles, rng)
    return Heap("small-blocks-4g", arena_bytes, off, size, live, h, "hash",
                0xC0FFEE00 + seed, seed)


def self_overlap_64gib(seed: int = 5, n_live: int = 64, block_bytes: int = 1 * GiB,
            hole_lo: int = 4 * KiB, hole_hi: int = 64 * MiB,
            n_handles: int = 1_000_000) -> Heap:
    """Self-overlap stress: n_live live blocks of block_bytes, each preceded by
    a freed hole of log-uniform hole_lo..hole_hi bytes (ceil to 32 B); the
    arena is exactly the sum (no tail).  Payload: u32 counter XOR seed."""
    rng = np.random.default_rng(seed)
    holes = _ceil_to(_loguniform(rng, hole_lo, hole_hi, n_live), 32)
    size = np.empty(2 * n_live, dtype=np.uint64)
    size[0::2] = holes
    size[1::2] = np.uint64(block_bytes)
    live = np.zeros(2 * n_live, dtype=np.uint8)
    live[1::2] = 1
    off = _packed_offsets(size)
    S = int(off[-1] + size[-1])
    h = draw_handles(off, size, live, n_handles, rng)
    return Heap("overlap-64g", S, off, size, live, h, "counter32",
                0x5EED0000 + seed, seed)


def small_shift_8gib(seed: int = 6, n_live: int = 8, block_bytes: int = 1 * GiB,
                     hole_lo: int = 4 * KiB, hole_hi: int = 1 * MiB,
                     n_handles: int = 1_000_000) -> Heap:
    """Small shifts: n_live live blocks of block_bytes, each above a freed hole
    of log-uniform hole_lo..hole_hi bytes (ceil to 32 B), so every block moves
    down by a few KiB to a few MiB -- far less than its size -- the regime
    where a tile most often waits for the one reading the bytes it
    overwrites.  Same layout as the self-overlap heap, with short holes."""
    rng = np.random.default_rng(seed)
    holes = _ceil_to(_loguniform(rng, hole_lo, hole_hi, n_live), 32)
    size = np.empty(2 * n_live, dtype=np.uint64)
    size[0::2] = holes
    size[1::2] = np.uint64(block_bytes)
    live = np.zeros(2 * n_live, dtype=np.uint8)
    live[1::2] = 1
    off = _packed_offsets(size)
    S = int(off[-1] + size[-1])
    h = draw_handles(off, size, live, n_handles, rng)
    return Heap("small-shift-8g", S, off, size, live, h, "hash", 0xC0FFEE00 + seed, seed)


# name -> (full size, reduced size with the same structure: small enough for
# the oracle to finish in seconds, large enough for several mover tiles)
_WORKLOADS = {
    "mixed-64m": (mixed_64mib,
                  lambda: mixed_64mib(n_blocks=1024, arena_bytes=16 * MiB, n_handles=4096)),
    "pairs-1g": (pairs_1gib,
                 lambda: pairs_1gib(n_pairs=2048, arena_bytes=64 * MiB, n_handles=65536)),
    "training-80g": (training_80gib,
                     lambda: training_80gib(arena_bytes=80 * 16 * MiB, n_small=3000, n_act=60,
                                            n_pinned=40, n_handles=65536)),
    "training-80g-pinned": (lambda: training_80gib(pin_params=True),
                            lambda: training_80gib(arena_bytes=80 * 16 * MiB, n_small=3000,
                                                   n_act=60, n_pinned=40, n_handles=65536,
                                                   pin_params=True)),
    "small-blocks-4g": (small_blocks_4gib,
                        lambda: small_blocks_4gib(n_blocks=60_000, arena_bytes=128 * MiB,
                                                  n_handles=65536)),
    "overlap-64g": (self_overlap_64gib,
                    lambda: self_overlap_64gib(n_live=8, block_bytes=8 * MiB, hole_lo=4 * KiB,
                                               hole_hi=1 * MiB, n_handles=65536)),
    "small-shift-8g": (small_shift_8gib,
                       lambda: small_shift_8gib(block_bytes=8 * MiB, hole_hi=64 * KiB,
                                                n_handles=65536)),
}
NAMES = tuple(_WORKLOADS)

# one line per workload, at its full size
SUMMARY = {
    "mixed-64m": "64 MiB arena, 4,096 blocks of 256 B-64 KiB, each live with p = 0.5; "
                 "16,384 handles",
    "pairs-1g": "1 GiB arena, 65,536 blocks as BF16/FP32-like pairs (b, 2b), live p = 0.6; "
                "1M handles",
    "training-80g": "80 GiB arena shaped like the 910C failure: 40 never-freed 1-2 GiB "
                    "parameter/optimizer blocks, 200 activation and 200k small blocks, "
                    "14 GiB free with free/largest - 1 = 4.7; 4M handles",
    "training-80g-pinned": "the 80 GiB training arena with its 40 parameter/optimizer "
                           "blocks pinned (immovable); 4M handles",
    "small-blocks-4g": "4 GiB arena, 2,000,000 blocks of 32-4,096 B alternating free/live "
                       "(every live block moves); 8M handles",
    "overlap-64g": "64 GiB arena of 64 live 1 GiB blocks, each above a freed 4 KiB-64 MiB "
                   "hole (every move self-overlapping); 1M handles",
    "small-shift-8g": "8 GiB arena of 8 live 1 GiB blocks, each above a freed 4 KiB-1 MiB "
                      "hole (every block shifts by a few KiB to a few MiB); 1M handles",
}


def workload(name: str, small: bool = False) -> Heap:
    """The named workload (a key of SUMMARY) at its full size, or its reduced
    variant with the same structure."""
    if name not in _WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; one of {', '.join(NAMES)}")
    full, reduced = _WORKLOADS[name]
    return reduced() if small else full()


# --------------------------------------------------------------------------
# tiny heaps for brute force
# --------------------------------------------------------------------------

def tiny_heap(rng: np.random.Generator, n: int, sizes=(32, 64, 96),
              gap_p: float = 0.3, tail_max: int = 3, live_p: float = 0.5,
              gran: int = 32, pinned_p: float = 0.0) -> Heap:
    """A small random table: n blocks with sizes from ``sizes``, optional
    untracked gaps (multiples of ``gran``) between them and an optional
    untracked tail."""
    size = np.array(rng.choice(sizes, n), dtype=np.uint64) if n else np.zeros(0, np.uint64)
    gaps = np.where(rng.random(n) < gap_p, rng.integers(1, 4, n), 0).astype(np.uint64) * np.uint64(gran)
    off = np.zeros(n, dtype=np.uint64)
    cur = 0
    for i in range(n):
        cur += int(gaps[i])
        off[i] = cur
        cur += int(size[i])
    S = cur + int(rng.integers(0, tail_max + 1)) * gran
    live = (rng.random(n) < live_p).astype(np.uint8)
    h = draw_handles(off, size, live, 4 * max(n, 1), rng)
    heap = Heap(f"tiny{n}", S, off, size, live, h, "hash", int(rng.integers(1, 1 << 62)), 0)
    if pinned_p > 0:
        heap.pinned = ((rng.random(n) < pinned_p) & (live == 1)).astype(np.uint8)
    heap.handles = np.concatenate([h, edge_handles(heap, rng, 8)])
    return heap


def table_from_lists(arena_bytes: int, blocks, live, handles=(), name="hand",
                     payload_mode="hash", payload_seed=7, pinned=None) -> Heap:
    """Build a Heap from explicit (offset, size) pairs, live and pinned flags."""
    off = np.array([b[0] for b in blocks], dtype=np.uint64)
    size = np.array([b[1] for b in blocks], dtype=np.uint64)
    lv = np.array(live, dtype=np.uint8)
    h = np.array(list(handles), dtype=np.uint64)
    heap = Heap(name, arena_bytes, off, size, lv, h, payload_mode, payload_seed, 0)
    if pinned is not None:
        heap.pinned = np.array(pinned, dtype=np.uint8)
    return heap

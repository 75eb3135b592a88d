"""Byte-level brute force for tiny heaps, written independently of the oracle.

Compaction is stated here as a stable partition of bytes inside each segment:
mark every byte of a movable live block; a segment is the span between two
pinned blocks (or an arena end); in each segment the marked bytes, in address
order, are written from the segment's start, and every other byte keeps its
value.  New offsets, holes and remapped handles are read off the byte maps by
counting, with no per-block running sum.  Only for arenas of a few MiB.
"""
import numpy as np

U64_MAX = (1 << 64) - 1


def _pin(pinned, n):
    return np.zeros(n, np.uint8) if pinned is None else pinned


def live_bitmap(arena_bytes, off, size, live):
    B = np.zeros(arena_bytes, dtype=bool)
    for o, s, l in zip(off.tolist(), size.tolist(), live.tolist()):
        if l:
            B[o:o + s] = True
    return B


def _maps(arena_bytes, off, size, live, pinned):
    """(movable-live byte map, pinned byte map, segment start of every byte)"""
    pinned = _pin(pinned, len(off))
    M = np.zeros(arena_bytes, dtype=bool)
    P = np.zeros(arena_bytes, dtype=bool)
    for o, s, l, p in zip(off.tolist(), size.tolist(), live.tolist(), pinned.tolist()):
        if p:
            P[o:o + s] = True
        elif l:
            M[o:o + s] = True
    seg = np.zeros(arena_bytes, dtype=np.int64)
    start = 0
    prev = False
    for a in range(arena_bytes):
        if prev and not P[a]:
            start = a                 # first byte after a pinned run
        seg[a] = start
        prev = bool(P[a])
    return M, P, seg


def compacted(arena, off, size, live, pinned=None):
    M, P, seg = _maps(arena.shape[0], off, size, live, pinned)
    out = arena.copy()
    S = arena.shape[0]
    a = 0
    while a < S:
        if P[a]:
            a += 1
            continue
        b = a
        while b < S and not P[b]:
            b += 1
        keep = arena[a:b][M[a:b]]
        out[a:a + keep.shape[0]] = keep
        a = b
    return out


def new_offsets(arena_bytes, off, size, live, pinned=None):
    M, P, seg = _maps(arena_bytes, off, size, live, pinned)
    below = np.concatenate([[0], np.cumsum(M, dtype=np.int64)])
    pinned = _pin(pinned, len(off))
    out = []
    for o, p in zip(off.tolist(), pinned.tolist()):
        if p:
            out.append(o)
        else:
            s0 = int(seg[o]) if o < arena_bytes else (int(seg[-1]) if arena_bytes else 0)
            out.append(s0 + int(below[o] - below[s0]))
    return np.array(out, dtype=np.uint64)


def holes(B):
    """Maximal runs of non-live bytes: list of (start, length)."""
    runs = []
    start = None
    for p, b in enumerate(B.tolist()):
        if not b and start is None:
            start = p
        elif b and start is not None:
            runs.append((start, p - start))
            start = None
    if start is not None:
        runs.append((start, len(B) - start))
    return runs


def stats(arena_bytes, off, size, live, pinned=None):
    B = live_bitmap(arena_bytes, off, size, live)
    hs = holes(B)
    lt = int(B.sum())
    F = arena_bytes - lt
    L = max((h[1] for h in hs), default=0)
    newo = new_offsets(arena_bytes, off, size, live, pinned)
    moved = [(i, int(size[i])) for i in range(len(off))
             if live[i] and int(newo[i]) != int(off[i])]
    r1 = 0.0 if F == 0 else F / L - 1.0
    r2 = 0.0 if F == 0 else 1.0 - L / F
    return dict(arena_bytes=arena_bytes, live_bytes=lt, free_bytes=F,
                largest_hole=L, hole_count=len(hs),
                live_blocks=int(np.count_nonzero(live)),
                moved_blocks=len(moved), moved_bytes=sum(s for _, s in moved),
                frag_free_over_largest_minus_1=r1,
                frag_one_minus_largest_over_free=r2)


def remap(arena_bytes, off, size, live, handles, pinned=None):
    M, P, seg = _maps(arena_bytes, off, size, live, pinned)
    rank = np.concatenate([[0], np.cumsum(M, dtype=np.int64)])
    out = []
    for h in handles.tolist():
        if h < arena_bytes and P[h]:
            out.append(h)
        elif h < arena_bytes and M[h]:
            s0 = int(seg[h])
            out.append(s0 + int(rank[h] - rank[s0]))
        else:
            out.append(U64_MAX)
    out = np.array(out, dtype=np.uint64)
    return out, int(np.count_nonzero(out == np.uint64(U64_MAX)))


def target_window(arena_bytes, off, size, live, request, pinned=None):
    """Targeted compaction by simulation.  Every window from the start of one
    hole to the end of the same or a later hole, holding no pinned byte, is
    tried on the byte map: its live bytes are packed to its start, the bytes
    whose address changed are counted, and the free run ending at the
    window's end is measured.  Among windows whose run holds `request` bytes,
    the fewest moved bytes wins, then the lowest start.
    Returns (found, begin, end, hole, moved)."""
    B = live_bitmap(arena_bytes, off, size, live)
    _, P, _ = _maps(arena_bytes, off, size, live, pinned)
    hs = holes(B)
    best = None
    for i in range(len(hs)):
        for j in range(i, len(hs)):
            a, b = hs[i][0], hs[j][0] + hs[j][1]
            if P[a:b].any():
                continue
            inside = B[a:b]
            k = int(inside.sum())
            packed = np.zeros(b - a, dtype=bool)
            packed[:k] = True
            last_live = int(np.flatnonzero(packed)[-1]) if k else -1
            run = (b - a) - (last_live + 1)
            if run < request:
                continue
            moved = int(np.count_nonzero(np.flatnonzero(inside) != np.arange(k)))
            key = (moved, a)
            if best is None or key < best[0]:
                best = (key, (1, a, b, run, moved))
    return best[1] if best else (0, 0, 0, 0, 0)


def first_fit(arena_bytes, off, size, live, request):
    """The pool of the CANN page (section 2.2) run on the byte map: round the
    request up to 32 bytes, list the free runs (merged neighbours) by
    address, take the first long enough.  U64_MAX if none."""
    need = -(-request // 32) * 32
    for start, length in holes(live_bitmap(arena_bytes, off, size, live)):
        if length >= need:
            return start
    return U64_MAX

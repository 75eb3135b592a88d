"""Byte-level brute force for tiny heaps, written independently of the oracle.

Compaction is stated here as a stable partition of bytes: mark every byte that
lies in a live block, then the compacted arena is the marked bytes in address
order followed by the original bytes from that point on.  New offsets, holes
and remapped handles are all read off the byte bitmap by counting, with no
per-block running sum.  Only for arenas of at most a few MiB.
"""
import numpy as np

U64_MAX = (1 << 64) - 1


def live_bitmap(arena_bytes, off, size, live):
    B = np.zeros(arena_bytes, dtype=bool)
    for o, s, l in zip(off.tolist(), size.tolist(), live.tolist()):
        if l:
            B[o:o + s] = True
    return B


def compacted(arena, B):
    out = arena.copy()
    keep = arena[B]
    out[:keep.shape[0]] = keep
    return out


def new_offsets(B, off):
    below = np.concatenate([[0], np.cumsum(B, dtype=np.int64)])
    return np.array([below[o] for o in off.tolist()], dtype=np.uint64)


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


def stats(arena_bytes, off, size, live):
    B = live_bitmap(arena_bytes, off, size, live)
    hs = holes(B)
    lt = int(B.sum())
    F = arena_bytes - lt
    L = max((h[1] for h in hs), default=0)
    newo = new_offsets(B, off)
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


def remap(arena_bytes, off, size, live, handles):
    B = live_bitmap(arena_bytes, off, size, live)
    rank = np.concatenate([[0], np.cumsum(B, dtype=np.int64)])
    out = []
    for h in handles.tolist():
        if h < arena_bytes and B[h]:
            out.append(int(rank[h]))
        else:
            out.append(U64_MAX)
    out = np.array(out, dtype=np.uint64)
    return out, int(np.count_nonzero(out == np.uint64(U64_MAX)))

// stats_one.h -- a statistics pass in one launch, as a device function, so
// that it can run in its own launch (plan.hip) or in the one-call path's
// remap launch (remap.hip).
//
// Page: "Ascend 910C cluster tuning", section "Total-usage monitoring misses
// fragmentation" (the free total and the largest contiguous free block);
// "CANN memory management and memory optimisation", section 3.2 (1 -
// largest/free) and section 2.2 (adjacent free blocks merge, so holes are
// maximal runs outside live blocks).
#ifndef ARENA_COMPACTION_STATS_ONE_H
#define ARENA_COMPACTION_STATS_ONE_H
#include "scan.h"

namespace ac {
namespace {

// ---------------------------------------------------------------------------
// A statistics pass in one launch (the post-check of a compaction).  Each
// workgroup summarises its chunk of entries on its own, with no prefix; the
// few quantities that depend on the entries before the chunk are kept
// apart:
//   * the hole below the chunk's first live block, which starts at the
//     highest live end before the chunk (a max over the chunks before);
//   * which of the chunk's blocks move.  A movable live block moves iff a
//     hole lies between the start of its segment's packed run and it.  A
//     block after a hole inside the chunk, or in a segment that starts
//     inside it (after a pinned block), is decided locally (`a`); the
//     blocks packed tight from the chunk's first live block, before any
//     pinned one (`b`), move iff the segment is *pending* there -- a hole
//     lies between the segment's start and that block, the hole just below
//     it included.  Pending passes from chunk to chunk: a chunk holding a
//     pinned block sets it to whether a hole follows its last pinned block;
//     any other chunk with live blocks ORs in its boundary hole and its
//     inner ones; an empty chunk passes it on.
// The last workgroup to finish (counted in the header; a plan run before
// clears the count) reads every summary, takes the max and the pending
// state across the (at most 1,024) chunks with two workgroup scans, and
// completes the header, which holds the same figures as the two-launch
// pass's.
struct ChunkSum {
    uint64_t cnt, lsum, mx, pcnt;  // live blocks, live bytes, highest live end (0: none), pinned
    uint64_t bad;                  // smallest bad-entry key
    uint64_t first;                // offset of the first live entry (kNone: none)
    uint64_t reset;                // a pinned entry is inside
    uint64_t pend;                 // reset: a hole follows the last pinned block; else a hole
                                   // follows the first live block
    uint64_t a_blocks, a_bytes;    // blocks that move whatever lies before the chunk
    uint64_t b_blocks, b_bytes;    // blocks that move iff pending at the first live block
    uint64_t max_gap, gaps;        // holes between live blocks inside the chunk
    uint64_t min_fit, min_size;
};
static_assert(sizeof(ChunkSum) == 16 * sizeof(uint64_t), "one 128-byte summary per chunk");

__device__ inline void csum_store(ChunkSum *p, const ChunkSum &c) {
    uint64_t *w = reinterpret_cast<uint64_t *>(p);
    const uint64_t *v = reinterpret_cast<const uint64_t *>(&c);
#pragma unroll
    for (int i = 0; i < 16; ++i) __hip_atomic_store(w + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t csum_field(const uint64_t *f) {
    return __hip_atomic_load(const_cast<uint64_t *>(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t max_op(uint64_t a, uint64_t b) { return umax64(a, b); }

// Exclusive workgroup scan of a u64 under max; also returns the total.
template <int NT>
__device__ inline uint64_t block_excl_max(uint64_t x, uint64_t &total, uint64_t *sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const uint64_t inc = wave_incl_scan(x, max_op);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if (k < w) pre = umax64(pre, sh[k]);
        tot = umax64(tot, sh[k]);
    }
    const uint64_t ex = wave_shift_up(inc);
    __syncthreads();
    total = tot;
    return umax64(pre, ex);
}

// The pending state as a function of the state before a chunk: constant
// (a pinned block inside sets it) or "or v" (bit 1: constant, bit 0: v).
// first then second:
__device__ inline uint32_t pend_then(uint32_t f, uint32_t g) {
    if (g & 2u) return g;
    return (f & 2u) | ((f | g) & 1u);
}

// Exclusive workgroup scan of pending functions (the identity is "or 0").
template <int NT>
__device__ inline uint32_t block_excl_pend(uint32_t x, uint32_t *sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(x, pend_then);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    uint32_t pre = 0u;
#pragma unroll
    for (int k = 0; k < NW; ++k)
        if (k < w) pre = pend_then(pre, sh[k]);
    const uint32_t ex = wave_shift_up(inc);
    __syncthreads();
    return pend_then(pre, ex);
}

// The pass as run by workgroup g (of NT lanes, ITEMS entries a lane per
// step) of at least `ngroups` workgroups taking part (those at or past it
// do nothing here): table t of n entries, chunks of `chunk` entries, the
// summaries in cs, the header hdr.  Workgroup-uniform; barriers inside.
template <int NT, int ITEMS = kScanItems>
__device__ void stats_one_part(const TableView &t, uint64_t n, uint64_t arena_bytes,
                               uint64_t chunk, uint64_t ngroups, ChunkSum *cs, WsHeader *hdr,
                               uint64_t fit_need, uint64_t g) {
    static_assert(NT % 64 == 0 && kMaxScanParts % NT == 0, "whole waves; whole chunks a lane");
    constexpr uint32_t kStep = NT * ITEMS;  // entries per workgroup step
    __shared__ Agg sh[kExclSlots<NT>];
    __shared__ uint64_t shr[NT / 64];
    __shared__ uint64_t s_red[kStatSlots<NT>];
    __shared__ uint32_t shp[NT / 64];
    __shared__ uint32_t s_last;
    if (g >= ngroups) return;
    const uint64_t base = g * chunk;
    const uint64_t end = umin64(base + chunk, n);
    const Window win = window_of(nullptr);
    Agg carry = agg_zero();  // this chunk's own, from zero
    uint64_t first = kNone;  // (workgroup-uniform)
    uint64_t bad = kNone, max_gap = 0, gaps = 0, min_fit = kNone, min_size = kNone;
    uint64_t a_blocks = 0, a_bytes = 0, b_blocks = 0, b_bytes = 0;
    for (uint64_t s0 = base; s0 < end; s0 += kStep) {
        const uint64_t i0 = s0 + (uint64_t)threadIdx.x * ITEMS;
        uint64_t o[ITEMS], s[ITEMS];
        uint32_t l[ITEMS], p[ITEMS], f[ITEMS];
        uint64_t prev_end = 0, my_first = kNone;
        if (i0 > 0 && i0 < n) prev_end = t.off[i0 - 1] + t.size[i0 - 1];
        Agg a = agg_zero();
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)ITEMS; ++k) {
            const uint64_t i = i0 + k;
            o[k] = s[k] = 0;
            l[k] = p[k] = f[k] = 0;
            if (i < n) {
                o[k] = t.off[i];
                s[k] = t.size[i];
                const uint32_t lr = live_of(t, i), pr = pin_of(t, i);  // as given: checked below
                l[k] = lr ? 1u : 0u;
                p[k] = pr ? 1u : 0u;
                f[k] = stays(o[k], l[k], p[k], win);
                const uint32_t r = entry_reason(i, o[k], s[k], lr, pr, arena_bytes, prev_end);
                if (r) bad = umin64(bad, (i << 3) | r);
                prev_end = o[k] + s[k];
                if (l[k] && my_first == kNone) my_first = o[k];
                a = combine(a, element(o[k], s[k], l[k], p[k], f[k]));
            }
        }
        // offsets ascend, so the chunk's first live entry has the least
        // offset among its live ones
        if (first == kNone) first = block_reduce<NT>(my_first, shr, OpMin());
        Agg tot;
        const Agg ex = block_excl<NT>(a, tot, sh);
        Agg run = combine(carry, ex);
        carry = combine(carry, tot);
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)ITEMS; ++k) {
            if (i0 + k >= n) continue;
            if (l[k]) {
                if (run.cnt) {  // the hole below this block lies inside the chunk
                    const uint64_t gap = o[k] - run.mx;
                    if (gap) {
                        gaps += 1;
                        max_gap = umax64(max_gap, gap);
                        if (gap >= fit_need) min_fit = umin64(min_fit, run.mx);
                    }
                }
                min_size = umin64(min_size, s[k]);
                if (!f[k]) {
                    if (run.r) {  // its segment starts inside the chunk: packed at run.v
                        if (o[k] != run.v) {
                            a_blocks += 1;
                            a_bytes += s[k];
                        }
                    } else if (o[k] - run.v != first) {  // a hole since the first live block
                        a_blocks += 1;
                        a_bytes += s[k];
                    } else {  // packed tight from the first live block
                        b_blocks += 1;
                        b_bytes += s[k];
                    }
                }
            }
            run = combine(run, element(o[k], s[k], l[k], p[k], f[k]));
        }
    }
    StatPart q{max_gap, gaps, a_blocks, a_bytes, bad, min_size, min_fit, 0};
    uint64_t x[4] = {b_blocks, b_bytes, 0, 0};
    block_reduce_stats<NT>(q, x, s_red);
    if (threadIdx.x == 0) {
        ChunkSum c;
        c.cnt = carry.cnt;
        c.lsum = carry.lsum;
        c.mx = carry.mx;
        c.pcnt = carry.pcnt;
        c.bad = q.min_moved_dst;  // (the bad key rode in that min slot)
        c.first = first;
        c.reset = carry.r ? 1u : 0u;
        c.pend = carry.r ? (carry.v < carry.mx ? 1u : 0u)
                         : (first != kNone && first + carry.v < carry.mx ? 1u : 0u);
        c.a_blocks = q.moved_blocks;
        c.a_bytes = q.moved_bytes;
        c.b_blocks = x[0];
        c.b_bytes = x[1];
        c.max_gap = q.max_gap;
        c.gaps = q.gaps;
        c.min_fit = q.min_fit;
        c.min_size = q.min_size;
        csum_store(cs + g, c);
        uint32_t last = 1;
        if (ngroups > 1) {
            // the summary's stores complete before the arrival is counted
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const uint64_t done = __hip_atomic_fetch_add(&hdr->arrive, 1ull, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            last = done + 1 == ngroups;
        }
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;

    // the last workgroup: chunks [threadIdx.x * kPer, + kPer).  A summary is
    // read in two parts -- the four fields the two scans need, then the rest
    // one chunk at a time while summing -- so no lane holds whole summaries.
    constexpr uint32_t kPer = kMaxScanParts / NT;
    const uint64_t j0 = (uint64_t)threadIdx.x * kPer;
    uint64_t mx_in[kPer], first_of[kPer];
    uint32_t rp[kPer];  // bit 1: a pinned entry inside; bit 0: its pend field
    uint64_t loc = 0;  // the highest live end before each chunk
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        uint64_t mx = 0, fi = kNone, re = 0, pe = 0;
        if (j0 + k < ngroups) {
            const ChunkSum *p = cs + j0 + k;
            mx = csum_field(&p->mx);
            fi = csum_field(&p->first);
            re = csum_field(&p->reset);
            pe = csum_field(&p->pend);
        }
        mx_in[k] = loc;
        loc = umax64(loc, mx);
        first_of[k] = fi;
        rp[k] = (re ? 2u : 0u) | (uint32_t)(pe & 1u);
    }
    uint64_t max_end;
    const uint64_t mx_ex = block_excl_max<NT>(loc, max_end, shr);
    // the hole below each chunk's first live block, and its pending function
    uint32_t fn[kPer], hole[kPer];
    uint32_t mine = 0u;  // this thread's chunks, composed
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        mx_in[k] = umax64(mx_in[k], mx_ex);
        hole[k] = (first_of[k] != kNone && mx_in[k] < first_of[k]) ? 1u : 0u;
        fn[k] = first_of[k] == kNone ? 0u : (rp[k] & 2u) ? rp[k] : ((hole[k] | rp[k]) & 1u);
        mine = pend_then(mine, fn[k]);
    }
    uint32_t pend = block_excl_pend<NT>(mine, shp) & 1u;  // state before chunk j0
    StatPart r{0, 0, 0, 0, kNone, kNone, kNone, 0};
    uint64_t tx[4] = {0, 0, 0, 0};  // live blocks, live bytes, pinned blocks
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        if (j0 + k >= ngroups) break;
        const ChunkSum *p = cs + j0 + k;
        const uint64_t pend_first = pend | hole[k];  // pending at the chunk's first live block
        r.moved_blocks += csum_field(&p->a_blocks) + (pend_first ? csum_field(&p->b_blocks) : 0);
        r.moved_bytes += csum_field(&p->a_bytes) + (pend_first ? csum_field(&p->b_bytes) : 0);
        r.gaps += csum_field(&p->gaps) + hole[k];
        r.max_gap = umax64(r.max_gap, csum_field(&p->max_gap));
        r.min_fit = umin64(r.min_fit, csum_field(&p->min_fit));
        if (hole[k]) {
            const uint64_t gap = first_of[k] - mx_in[k];
            r.max_gap = umax64(r.max_gap, gap);
            if (gap >= fit_need) r.min_fit = umin64(r.min_fit, mx_in[k]);
        }
        r.min_moved_dst = umin64(r.min_moved_dst, csum_field(&p->bad));
        r.min_size = umin64(r.min_size, csum_field(&p->min_size));
        tx[0] += csum_field(&p->cnt);
        tx[1] += csum_field(&p->lsum);
        tx[2] += csum_field(&p->pcnt);
        pend = pend_then(pend, fn[k]) & 1u;
    }
    block_reduce_stats<NT>(r, tx, s_red);
    if (threadIdx.x == 0) {
        hdr->live_bytes = tx[1];
        hdr->max_live_end = max_end;
        hdr->live_blocks = tx[0];
        hdr->pinned_blocks = tx[2];
        hdr->bad_key = r.min_moved_dst;
        hdr->win_state = kWinNone;
        const uint64_t tail = arena_bytes - max_end;
        uint64_t fit = r.min_fit;
        // holes below live blocks come first in address order; the tail last
        if (fit == kNone && tail && tail >= fit_need) fit = max_end;
        hdr->fit_offset = fit;
        hdr->largest_hole = umax64(r.max_gap, tail);
        hdr->hole_count = r.gaps + (tail ? 1 : 0);
        hdr->moved_blocks = r.moved_blocks;
        hdr->moved_bytes = r.moved_bytes;
        hdr->small_moved = 0;
        hdr->min_live_size = r.min_size;
        hdr->move_begin = kNone;
        hdr->arrive = 0;  // every pass leaves it cleared
    }
}

}  // namespace
}  // namespace ac

#endif

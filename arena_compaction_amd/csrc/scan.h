// scan.h -- device primitives of the table scans, shared by the plan's
// passes and the one-launch statistics pass (included by plan.hip and
// remap.hip, each taking its own copy).
//
// Page: "Ascend 910C cluster tuning: memory-fragment compaction in
// mixed-precision training", section "Periodic compaction with Ascend C":
// holes are scanned from low to high addresses and each live tensor gets the
// downward shift it needs; section "Cutting alloc and free at the source":
// a pinned entry stays put and splits the arena into segments that pack
// independently.  The scan state (Agg) is, per prefix of the table:
//   v    : packed position, reset to a pinned entry's end (segmented sum)
//   mx   : max end of the live entries so far
//   cnt  : live entries so far (index into the packed live arrays)
//   lsum : live bytes so far;   pcnt: pinned entries so far
#ifndef ARENA_COMPACTION_SCAN_H
#define ARENA_COMPACTION_SCAN_H
#include "internal.h"
#include "wave.h"

namespace ac {
namespace {

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ inline Agg agg_zero() { return Agg{0, 0, 0, 0, 0, 0, 0}; }

// Associative, not commutative: a before b.
__device__ inline Agg combine(const Agg &a, const Agg &b) {
    Agg c;
    c.r = a.r | b.r;
    c.v = b.r ? b.v : a.v + b.v;
    c.mx = umax64(a.mx, b.mx);
    c.cnt = a.cnt + b.cnt;
    c.lsum = a.lsum + b.lsum;
    c.pcnt = a.pcnt + b.pcnt;
    c.pad = 0;
    return c;
}

// p: the entry is pinned; f: it stays in place (pinned, or a live block
// outside a targeted plan's window).  A block that stays starts a segment.
__device__ inline Agg element(uint64_t o, uint64_t s, uint32_t l, uint32_t p, uint32_t f) {
    Agg e = agg_zero();
    if (f) {
        e.r = 1;
        e.v = o + s;
    } else if (l) {
        e.v = s;
    }
    if (l) {
        e.mx = o + s;
        e.cnt = 1;
        e.lsum = s;
    }
    e.pcnt = p;
    return e;
}

// One step of a wave scan over Agg: combine() with the value the DPP
// control brings from another lane before this lane's, a field at a time.
// Each field of the combined state depends only on that field of both
// sides (v also on this lane's r), so only one field's cross-lane
// temporaries are live at once, which keeps the side job's 1,024-lane mover
// under its register cap.  A lane with no source takes the identity (zero).
template <int CTRL, int ROW_MASK>
__device__ inline void agg_step(Agg &x) {
    const uint32_t ar = dpp_move<CTRL, ROW_MASK>(x.r);
    const uint64_t av = dpp_move<CTRL, ROW_MASK>(x.v);
    x.v = x.r ? x.v : av + x.v;
    x.r |= ar;
    x.mx = umax64(dpp_move<CTRL, ROW_MASK>(x.mx), x.mx);
    x.cnt += dpp_move<CTRL, ROW_MASK>(x.cnt);
    x.lsum += dpp_move<CTRL, ROW_MASK>(x.lsum);
    x.pcnt += dpp_move<CTRL, ROW_MASK>(x.pcnt);
}

// wave_incl_scan (wave.h) over Agg under combine(), by agg_step.
template <int SPAN = 64>
__device__ inline Agg agg_incl_scan(Agg x) {
    static_assert(SPAN == 64 || (SPAN >= 1 && SPAN <= 16), "a whole wave or one row");
    if constexpr (SPAN > 1) agg_step<kDppRowShr | 1, 0xf>(x);
    if constexpr (SPAN > 2) agg_step<kDppRowShr | 2, 0xf>(x);
    if constexpr (SPAN > 4) agg_step<kDppRowShr | 4, 0xf>(x);
    if constexpr (SPAN > 8) agg_step<kDppRowShr | 8, 0xf>(x);
    if constexpr (SPAN > 16) {
        agg_step<kDppRowBcast15, 0xa>(x);  // rows 1, 3 after rows 0, 2
        agg_step<kDppRowBcast31, 0xc>(x);  // rows 2, 3 after rows 0-1
    }
    return x;
}

// The lane before's value (the identity in lane 0), a field at a time.
__device__ inline Agg agg_shift_up(const Agg &x) {
    Agg y;
    y.v = wave_shift_up(x.v);
    y.mx = wave_shift_up(x.mx);
    y.cnt = wave_shift_up(x.cnt);
    y.lsum = wave_shift_up(x.lsum);
    y.pcnt = wave_shift_up(x.pcnt);
    y.r = wave_shift_up(x.r);
    y.pad = 0;
    return y;
}

// LDS slots the two cross-wave helpers below need for NT lanes.
template <int NT>
constexpr int kExclSlots = 2 * (NT / 64) + 1;  // Agg slots of block_excl
template <int NT>
constexpr int kStatSlots = 12 * (NT / 64 + 1);  // u64 slots of block_reduce_stats

// Exclusive workgroup scan in thread order; also returns the total.
// sh: kExclSlots<NT> entries.  Each wave scans itself across its lanes; the
// first wave then scans the waves' totals (one per lane) and hands every
// wave its prefix through LDS, so no lane holds more than a few aggregates.
template <int NT>
__device__ inline Agg block_excl(const Agg &x, Agg &total, Agg *sh) {
    constexpr int NW = NT / 64;
    static_assert(NW >= 1 && NW <= 16 && (NW & (NW - 1)) == 0, "whole waves, a power of two");
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const Agg inc = agg_incl_scan(x);
    const Agg ex = agg_shift_up(inc);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
        const Agg t = agg_incl_scan<NW>(lane < NW ? sh[lane] : agg_zero());
        const Agg te = agg_shift_up(t);
        if (lane < NW) sh[NW + lane] = te;
        if (lane == NW - 1) sh[2 * NW] = t;
    }
    __syncthreads();
    const Agg pre = wave_uniform(sh[NW + w]);  // the wave's prefix
    total = wave_uniform(sh[2 * NW]);
    __syncthreads();
    return combine(pre, ex);
}

__device__ inline uint64_t add_op(uint64_t a, uint64_t b) { return a + b; }

// Exclusive workgroup sum of u64; also returns the total.  sh: NT/64 slots.
template <int NT>
__device__ inline uint64_t block_excl_sum(uint64_t x, uint64_t &total, uint64_t *sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const uint64_t inc = wave_incl_scan(x, add_op);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if (k < w) pre += sh[k];
        tot += sh[k];
    }
    const uint64_t ex = wave_shift_up(inc);
    __syncthreads();
    total = tot;
    return pre + ex;
}

// Workgroup reductions through LDS (NT threads, sh has NT/64 slots).
template <int NT, typename Op>
__device__ inline uint64_t block_reduce(uint64_t v, uint64_t *sh, Op op) {
    constexpr int NW = NT / 64;
    v = wave_reduce(v, op);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) r = op(r, sh[k]);
    __syncthreads();
    return wave_uniform(r);
}

struct OpAdd { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; } };
struct OpMax { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return umax64(a, b); } };
struct OpMin { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return umin64(a, b); } };

// The statistics and up to four extra sums, as one value to reduce.
struct StatRow {
    StatPart q;
    uint64_t x[4];
};
__device__ inline void stat_store(uint64_t *o, const StatRow &r) {
    o[0] = r.q.max_gap; o[1] = r.q.gaps; o[2] = r.q.moved_blocks; o[3] = r.q.moved_bytes;
    o[4] = r.q.min_moved_dst; o[5] = r.q.min_size; o[6] = r.q.min_fit; o[7] = r.q.small_moved;
    o[8] = r.x[0]; o[9] = r.x[1]; o[10] = r.x[2]; o[11] = r.x[3];
}
__device__ inline StatRow stat_load(const uint64_t *o) {
    return StatRow{StatPart{o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]},
                   {o[8], o[9], o[10], o[11]}};
}

// The row reduced over the first SPAN lanes of the wave (wave_reduce's
// SPAN), one field at a time: a field's cross-lane temporaries are live
// only while it is reduced, which keeps the side job's 1,024-lane mover
// under its register cap.
template <int SPAN = 64>
__device__ inline StatRow wave_reduce_row(const StatRow &r) {
    StatRow o;
    o.q.max_gap = wave_reduce<SPAN>(r.q.max_gap, umax64);
    o.q.gaps = wave_reduce<SPAN>(r.q.gaps, add_op);
    o.q.moved_blocks = wave_reduce<SPAN>(r.q.moved_blocks, add_op);
    o.q.moved_bytes = wave_reduce<SPAN>(r.q.moved_bytes, add_op);
    o.q.min_moved_dst = wave_reduce<SPAN>(r.q.min_moved_dst, umin64);
    o.q.min_size = wave_reduce<SPAN>(r.q.min_size, umin64);
    o.q.min_fit = wave_reduce<SPAN>(r.q.min_fit, umin64);
    o.q.small_moved = wave_reduce<SPAN>(r.q.small_moved, add_op);
#pragma unroll
    for (int k = 0; k < 4; ++k) o.x[k] = wave_reduce<SPAN>(r.x[k], add_op);
    return o;
}

// Workgroup reduction of the statistics and up to four extra sums: each
// wave reduces across its lanes and writes one row to LDS; the first wave's
// lanes take one row each and reduce them the same way; every lane reads
// the result.  sh: kStatSlots<NT> slots.
template <int NT>
__device__ inline void block_reduce_stats(StatPart &q, uint64_t (&x)[4], uint64_t *sh) {
    constexpr int NW = NT / 64;
    static_assert(NW >= 1 && NW <= 16 && (NW & (NW - 1)) == 0, "whole waves, a power of two");
    constexpr int F = 12;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const StatRow r = wave_reduce_row(StatRow{q, {x[0], x[1], x[2], x[3]}});
    if (lane == 0) stat_store(sh + F * w, r);
    __syncthreads();
    if (w == 0) {
        const StatRow t = wave_reduce_row<NW>(stat_load(sh + F * (lane < NW ? lane : 0)));
        if (lane == 0) stat_store(sh + F * NW, t);
    }
    __syncthreads();
    const StatRow t = wave_uniform(stat_load(sh + F * NW));
    q = t.q;
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = t.x[k];
    __syncthreads();
}

// Reason code of entry i (0 when it passes); checks in the documented order.
__device__ inline uint32_t entry_reason(uint64_t i, uint64_t o, uint64_t s, uint32_t l,
                                        uint32_t p, uint64_t arena_bytes, uint64_t prev_end) {
    if (s == 0) return 1;
    if ((o | s) & 31u) return 2;
    if (l > 1u) return 3;
    if (p > 1u || (p == 1u && l == 0u)) return 7;
    if (o > arena_bytes || s > arena_bytes - o) return 4;
    if (i > 0 && prev_end > o) return 5;
    return 0;
}

__device__ inline uint32_t live_of(const TableView &t, uint64_t i) { return t.live ? t.live[i] : 1u; }
__device__ inline uint32_t pin_of(const TableView &t, uint64_t i) { return t.pinned ? t.pinned[i] : 0u; }

// A targeted plan moves only the live blocks inside its window [begin, end);
// win is null for a full plan.
struct Window {
    uint64_t begin, end;
};
__device__ inline Window window_of(const uint64_t *win) {
    return win ? Window{win[0], win[1]} : Window{0, kNone};
}
__device__ inline uint32_t stays(uint64_t o, uint32_t l, uint32_t p, const Window &w) {
    return (p || (l && (o < w.begin || o >= w.end))) ? 1u : 0u;
}

}  // namespace
}  // namespace ac

#endif

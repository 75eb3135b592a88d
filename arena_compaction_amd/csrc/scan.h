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

__device__ inline Agg shfl_up_agg(const Agg &a, int d) {
    Agg b;
    b.v = __shfl_up(a.v, d, 64);
    b.mx = __shfl_up(a.mx, d, 64);
    b.cnt = __shfl_up(a.cnt, d, 64);
    b.lsum = __shfl_up(a.lsum, d, 64);
    b.pcnt = __shfl_up(a.pcnt, d, 64);
    b.r = __shfl_up(a.r, d, 64);
    b.pad = 0;
    return b;
}

// LDS slots the two cross-wave helpers below need for NT lanes.
template <int NT>
constexpr int kExclSlots = 2 * (NT / 64) + 1;  // Agg slots of block_excl
template <int NT>
constexpr int kStatSlots = 12 * (NT / 64 + 1);  // u64 slots of block_reduce_stats

// Exclusive workgroup scan in thread order; also returns the total.
// sh: kExclSlots<NT> entries.  Each wave scans itself with shuffles; the
// first wave then scans the waves' totals (one per lane) and hands every
// wave its prefix through LDS, so no lane holds more than a few aggregates.
template <int NT>
__device__ inline Agg block_excl(const Agg &x, Agg &total, Agg *sh) {
    constexpr int NW = NT / 64;
    static_assert(NW >= 1 && NW <= 64 && (NW & (NW - 1)) == 0, "whole waves, a power of two");
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    Agg inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const Agg y = shfl_up_agg(inc, d);
        if (lane >= d) inc = combine(y, inc);
    }
    Agg ex = shfl_up_agg(inc, 1);
    if (lane == 0) ex = agg_zero();
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    if (w == 0) {
        Agg t = lane < NW ? sh[lane] : agg_zero();
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            const Agg y = shfl_up_agg(t, d);
            if (lane >= d) t = combine(y, t);
        }
        Agg te = shfl_up_agg(t, 1);
        if (lane == 0) te = agg_zero();
        if (lane < NW) sh[NW + lane] = te;
        if (lane == NW - 1) sh[2 * NW] = t;
    }
    __syncthreads();
    const Agg pre = sh[NW + w];
    total = sh[2 * NW];
    __syncthreads();
    return combine(pre, ex);
}

// Exclusive workgroup sum of u64; also returns the total.  sh: NT/64 slots.
template <int NT>
__device__ inline uint64_t block_excl_sum(uint64_t x, uint64_t &total, uint64_t *sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    uint64_t inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
    }
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    uint64_t pre = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if (k < w) pre += sh[k];
        tot += sh[k];
    }
    uint64_t ex = __shfl_up(inc, 1, 64);
    if (lane == 0) ex = 0;
    __syncthreads();
    total = tot;
    return pre + ex;
}

// Workgroup reductions through LDS (NT threads, sh has NT/64 slots).
template <int NT, typename Op>
__device__ inline uint64_t block_reduce(uint64_t v, uint64_t *sh, Op op) {
    constexpr int NW = NT / 64;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = op(v, (uint64_t)__shfl_xor(v, d, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) r = op(r, sh[k]);
    __syncthreads();
    return r;
}

struct OpAdd { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; } };
struct OpMax { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return umax64(a, b); } };
struct OpMin { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return umin64(a, b); } };

// Workgroup reduction of the statistics and up to four extra sums: each
// wave reduces with shuffles and writes one row to LDS; the first wave's
// lanes take one row each and reduce them with shuffles; every lane reads
// the result.  sh: kStatSlots<NT> slots.
__device__ inline void stat_shfl_reduce(StatPart &q, uint64_t (&x)[4], int d) {
    q.max_gap = umax64(q.max_gap, (uint64_t)__shfl_xor(q.max_gap, d, 64));
    q.gaps += (uint64_t)__shfl_xor(q.gaps, d, 64);
    q.moved_blocks += (uint64_t)__shfl_xor(q.moved_blocks, d, 64);
    q.moved_bytes += (uint64_t)__shfl_xor(q.moved_bytes, d, 64);
    q.min_moved_dst = umin64(q.min_moved_dst, (uint64_t)__shfl_xor(q.min_moved_dst, d, 64));
    q.min_size = umin64(q.min_size, (uint64_t)__shfl_xor(q.min_size, d, 64));
    q.min_fit = umin64(q.min_fit, (uint64_t)__shfl_xor(q.min_fit, d, 64));
    q.small_moved += (uint64_t)__shfl_xor(q.small_moved, d, 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] += (uint64_t)__shfl_xor(x[k], d, 64);
}
__device__ inline void stat_store(uint64_t *o, const StatPart &q, const uint64_t (&x)[4]) {
    o[0] = q.max_gap; o[1] = q.gaps; o[2] = q.moved_blocks; o[3] = q.moved_bytes;
    o[4] = q.min_moved_dst; o[5] = q.min_size; o[6] = q.min_fit; o[7] = q.small_moved;
    o[8] = x[0]; o[9] = x[1]; o[10] = x[2]; o[11] = x[3];
}
__device__ inline void stat_load(const uint64_t *o, StatPart &q, uint64_t (&x)[4]) {
    q = StatPart{o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
    x[0] = o[8]; x[1] = o[9]; x[2] = o[10]; x[3] = o[11];
}
template <int NT>
__device__ inline void block_reduce_stats(StatPart &q, uint64_t (&x)[4], uint64_t *sh) {
    constexpr int NW = NT / 64;
    static_assert(NW >= 1 && NW <= 64 && (NW & (NW - 1)) == 0, "whole waves, a power of two");
    constexpr int F = 12;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) stat_shfl_reduce(q, x, d);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    if (lane == 0) stat_store(sh + F * w, q, x);
    __syncthreads();
    if (w == 0) {
        if (lane < NW) {
            stat_load(sh + F * lane, q, x);
        } else {  // the identity
            q = StatPart{0, 0, 0, 0, kNone, kNone, kNone, 0};
            x[0] = x[1] = x[2] = x[3] = 0;
        }
#pragma unroll
        for (int d = NW / 2; d >= 1; d >>= 1) stat_shfl_reduce(q, x, d);
        if (lane == 0) stat_store(sh + F * NW, q, x);
    }
    __syncthreads();
    stat_load(sh + F * NW, q, x);
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

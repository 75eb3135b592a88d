// plan.hip -- validation, live-size scan, hole statistics and the mover's tile
// table, for gfx950 (wave64).
//
// Page: "Ascend 910C cluster tuning: memory-fragment compaction in
// mixed-precision training", section "Periodic compaction with Ascend C":
// holes are scanned from low to high addresses and each live tensor gets the
// downward shift it needs.  Section "Cutting alloc and free at the source" of
// the same page keeps the parameter region at fixed addresses: a pinned entry
// stays put and splits the arena into segments that pack independently.
// Here all of it is one exclusive scan over the table of
//   v    : packed position, reset to a pinned entry's end (segmented sum)
//   mx   : max end of the live entries so far
//   cnt  : live entries so far (index into the packed live arrays)
//   lsum : live bytes so far;   pcnt: pinned entries so far
// so that
//   new offset of entry i   = offset_i if pinned, else v before i
//   hole just below live i  = offset_i - (mx before i)
// Section "Total-usage monitoring misses fragmentation" of the same page asks
// for the free total and the largest contiguous free block; section 3.2 of
// "CANN memory management and memory optimisation" defines the ratio
// 1 - largest/free.  Holes are maximal runs outside live blocks (the CANN pool
// merges adjacent free blocks, section 2.2), so one pass over live entries in
// order sees every hole once, plus the tail above the highest live block.
//
// Passes (n up to 2^32 entries): per-workgroup aggregates, a single-workgroup
// spine scan, a downsweep that writes new offsets, the packed live-block
// arrays (new and old offset, size, pinned flag) and per-workgroup
// statistics, and a single-workgroup finish.  Then the mover's tiles: every
// moved block counts the tiles that start inside it (a run of moved blocks
// starts one, and so does every tile-size boundary inside a run), and the
// remap's bucket index over old offsets is built (it also narrows the tiles'
// source searches) -- in a plan the finish, these counts and the index share
// one launch, as each reads only what the scan wrote; a scan of the counts
// gives each block its first tile, and one lane per tile writes the tile's
// start, its range, its blocks and its dependencies.  The whole sequence is
// queued at once; the host reads the header back only at the end.
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

// Exclusive workgroup scan in thread order; also returns the total.
// sh needs NT/64 entries.
template <int NT>
__device__ inline Agg block_excl(const Agg &x, Agg &total, Agg *sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    Agg inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const Agg y = shfl_up_agg(inc, d);
        if (lane >= d) inc = combine(y, inc);
    }
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    Agg pre = agg_zero(), tot = agg_zero();
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const Agg z = sh[k];
        if (k < w) pre = combine(pre, z);
        tot = combine(tot, z);
    }
    Agg ex = shfl_up_agg(inc, 1);
    if (lane == 0) ex = agg_zero();
    __syncthreads();
    total = tot;
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

// Nothing more to plan: the table is invalid, or no window fits the request.
__device__ inline bool plan_dead(const WsHeader *hdr) {
    return hdr->bad_key != kNone || hdr->win_state == kWinNoFit;
}

// Pass 1: per-workgroup aggregate and first bad key.  Workgroup g takes the
// entries [g * chunk, (g + 1) * chunk), kScanTile at a time.
__global__ __launch_bounds__(kScanThreads) void k_scan_partials(TableView t, uint64_t arena_bytes,
                                                                const uint64_t *win,
                                                                uint64_t chunk, ScanPart *part) {
    __shared__ Agg sh[kScanThreads / 64];
    __shared__ uint64_t shr[kScanThreads / 64];
    const Window w = window_of(win);
    const uint64_t base = (uint64_t)blockIdx.x * chunk;
    const uint64_t end = umin64(base + chunk, t.n);
    Agg acc = agg_zero();
    uint64_t bad = kNone;
    for (uint64_t s0 = base; s0 < end; s0 += kScanTile) {
        const uint64_t i0 = s0 + (uint64_t)threadIdx.x * kScanItems;
        Agg a = agg_zero();
        uint64_t prev_end = 0;
        if (i0 > 0 && i0 < t.n) prev_end = t.off[i0 - 1] + t.size[i0 - 1];
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            if (i < t.n) {
                const uint64_t o = t.off[i], s = t.size[i];
                const uint32_t l = live_of(t, i), p = pin_of(t, i);
                const uint32_t r = entry_reason(i, o, s, l, p, arena_bytes, prev_end);
                if (r) bad = umin64(bad, (i << 3) | r);
                const uint32_t lb = l ? 1u : 0u, pb = p ? 1u : 0u;
                a = combine(a, element(o, s, lb, pb, stays(o, lb, pb, w)));
                prev_end = o + s;
            }
        }
        Agg total;
        block_excl<kScanThreads>(a, total, sh);
        acc = combine(acc, total);
    }
    bad = block_reduce<kScanThreads>(bad, shr, OpMin());
    if (threadIdx.x == 0) part[blockIdx.x] = ScanPart{acc, bad};
}

// Pass 2 (one workgroup): exclusive scan of the aggregates; table totals.
__global__ __launch_bounds__(kSpineThreads) void k_scan_spine(const ScanPart *part, ScanPart *prefix,
                                                              uint64_t nb, WsHeader *hdr,
                                                              int reset_window) {
    __shared__ Agg sh[kSpineThreads / 64];
    __shared__ uint64_t shr[kSpineThreads / 64];
    Agg carry = agg_zero();
    uint64_t bad = kNone;
    for (uint64_t base = 0; base < nb; base += kSpineThreads) {
        const uint64_t j = base + threadIdx.x;
        Agg x = agg_zero();
        if (j < nb) {
            x = part[j].a;
            bad = umin64(bad, part[j].bad_key);
        }
        Agg total;
        const Agg ex = block_excl<kSpineThreads>(x, total, sh);
        if (j < nb) prefix[j] = ScanPart{combine(carry, ex), 0};
        carry = combine(carry, total);
    }
    bad = block_reduce<kSpineThreads>(bad, shr, OpMin());
    if (threadIdx.x == 0) {
        hdr->live_bytes = carry.lsum;
        hdr->max_live_end = carry.mx;
        hdr->live_blocks = carry.cnt;
        hdr->pinned_blocks = carry.pcnt;
        hdr->bad_key = bad;
        if (reset_window) hdr->win_state = kWinNone;
    }
}

struct LiveOut {
    uint64_t *dst, *src, *size;
    uint8_t *pin;
    uint64_t *z;   // live bytes below each live block (selection only)
    uint32_t *pc;  // pinned blocks below each live block (selection only)
    LiveRec *rec;      // the remap's (old end, shift) per live block, or
    LiveRec32 *rec32;  // the same in 32-byte units (arenas below 2^37 bytes)
    RemapEnt *ent;     // or key and 32-bit record together (then rec, rec32, key null)
    uint32_t *key;      // the remap's 32-bit search keys (null: 64-bit offsets)
    uint64_t key_mask;  // old offset -> offset inside its remap bucket
};

// Pass 3: new offsets, packed live arrays, per-workgroup hole/move stats.
__global__ __launch_bounds__(kScanThreads) void k_scan_down(TableView t, const uint64_t *win,
                                                            const ScanPart *prefix,
                                                            const WsHeader *hdr, uint64_t *new_offset,
                                                            LiveOut lo, StatPart *spart,
                                                            int outputs, uint64_t fit_need,
                                                            uint64_t chunk) {
    __shared__ Agg sh[kScanThreads / 64];
    __shared__ uint64_t shr[kScanThreads / 64];
    if (plan_dead(hdr)) return;  // invalid table or nothing to plan: write nothing
    const Window w = window_of(win);
    const uint64_t base = (uint64_t)blockIdx.x * chunk;
    const uint64_t end = umin64(base + chunk, t.n);
    Agg carry = prefix[blockIdx.x].a;  // everything before this workgroup's chunk
    uint64_t max_gap = 0, gaps = 0, moved = 0, moved_bytes = 0, min_dst = kNone, min_size = kNone;
    uint64_t min_fit = kNone, small_moved = 0;
    for (uint64_t s0 = base; s0 < end; s0 += kScanTile) {
        const uint64_t i0 = s0 + (uint64_t)threadIdx.x * kScanItems;
        uint64_t o[kScanItems], s[kScanItems];
        uint32_t l[kScanItems], p[kScanItems], f[kScanItems];
        Agg a = agg_zero();
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            o[k] = 0;
            s[k] = 0;
            l[k] = 0;
            p[k] = 0;
            f[k] = 0;
            if (i < t.n) {
                o[k] = t.off[i];
                s[k] = t.size[i];
                l[k] = live_of(t, i) ? 1u : 0u;
                p[k] = pin_of(t, i) ? 1u : 0u;
                f[k] = stays(o[k], l[k], p[k], w);
                a = combine(a, element(o[k], s[k], l[k], p[k], f[k]));
            }
        }
        Agg total;
        const Agg ex = block_excl<kScanThreads>(a, total, sh);
        Agg run = combine(carry, ex);
        carry = combine(carry, total);
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            if (i < t.n) {
                const uint64_t nw = f[k] ? o[k] : run.v;
                if ((outputs & kOutNew) && new_offset) new_offset[i] = nw;
                if (l[k]) {
                    if (outputs & kOutNew) {
                        lo.dst[run.cnt] = nw;
                        lo.pin[run.cnt] = (uint8_t)p[k];
                        if (lo.ent)
                            lo.ent[run.cnt] = RemapEnt{(uint32_t)(o[k] & lo.key_mask),
                                                       (uint32_t)((o[k] + s[k]) >> 5),
                                                       (uint32_t)((o[k] - nw) >> 5), 0u};
                        else if (lo.rec32)
                            lo.rec32[run.cnt] = LiveRec32{(uint32_t)((o[k] + s[k]) >> 5),
                                                          (uint32_t)((o[k] - nw) >> 5)};
                        else
                            lo.rec[run.cnt] = LiveRec{o[k] + s[k], o[k] - nw};
                        if (lo.key) lo.key[run.cnt] = (uint32_t)(o[k] & lo.key_mask);
                    }
                    if (outputs & (kOutNew | kOutSelect)) {
                        lo.src[run.cnt] = o[k];
                        lo.size[run.cnt] = s[k];
                    }
                    if (outputs & kOutSelect) {
                        lo.z[run.cnt] = run.lsum;
                        lo.pc[run.cnt] = (uint32_t)run.pcnt;
                    }
                    const uint64_t gap = o[k] - run.mx;
                    if (gap) {
                        gaps += 1;
                        max_gap = umax64(max_gap, gap);
                        if (gap >= fit_need) min_fit = umin64(min_fit, run.mx);
                    }
                    if (o[k] != nw) {
                        moved += 1;
                        moved_bytes += s[k];
                        min_dst = umin64(min_dst, nw);
                        if (o[k] - nw < kAutoSmallShift) small_moved += s[k];
                    }
                    min_size = umin64(min_size, s[k]);
                }
                run = combine(run, element(o[k], s[k], l[k], p[k], f[k]));
            }
        }
    }  // steps of the chunk
    max_gap = block_reduce<kScanThreads>(max_gap, shr, OpMax());
    gaps = block_reduce<kScanThreads>(gaps, shr, OpAdd());
    moved = block_reduce<kScanThreads>(moved, shr, OpAdd());
    moved_bytes = block_reduce<kScanThreads>(moved_bytes, shr, OpAdd());
    min_dst = block_reduce<kScanThreads>(min_dst, shr, OpMin());
    min_size = block_reduce<kScanThreads>(min_size, shr, OpMin());
    min_fit = block_reduce<kScanThreads>(min_fit, shr, OpMin());
    small_moved = block_reduce<kScanThreads>(small_moved, shr, OpAdd());
    if (threadIdx.x == 0)
        spart[blockIdx.x] =
            StatPart{max_gap, gaps, moved, moved_bytes, min_dst, min_size, min_fit, small_moved};
}

// Pass 4 (one workgroup): reduce the statistics, add the tail hole.  A plan
// runs it inside the launch after the scan (k_after_scan); a statistics pass
// alone launches it by itself.
__device__ void scan_finish(const StatPart *spart, uint64_t nb, uint64_t arena_bytes,
                            WsHeader *hdr, int outputs, uint64_t epoch, uint64_t fit_need) {
    __shared__ uint64_t sh[kSpineThreads / 64];
    if (plan_dead(hdr)) return;
    uint64_t max_gap = 0, gaps = 0, moved = 0, moved_bytes = 0, min_dst = kNone, min_size = kNone;
    uint64_t min_fit = kNone, small_moved = 0;
    for (uint64_t j = threadIdx.x; j < nb; j += kSpineThreads) {
        const StatPart q = spart[j];
        small_moved += q.small_moved;
        min_fit = umin64(min_fit, q.min_fit);
        max_gap = umax64(max_gap, q.max_gap);
        gaps += q.gaps;
        moved += q.moved_blocks;
        moved_bytes += q.moved_bytes;
        min_dst = umin64(min_dst, q.min_moved_dst);
        min_size = umin64(min_size, q.min_size);
    }
    max_gap = block_reduce<kSpineThreads>(max_gap, sh, OpMax());
    gaps = block_reduce<kSpineThreads>(gaps, sh, OpAdd());
    moved = block_reduce<kSpineThreads>(moved, sh, OpAdd());
    moved_bytes = block_reduce<kSpineThreads>(moved_bytes, sh, OpAdd());
    min_dst = block_reduce<kSpineThreads>(min_dst, sh, OpMin());
    min_size = block_reduce<kSpineThreads>(min_size, sh, OpMin());
    min_fit = block_reduce<kSpineThreads>(min_fit, sh, OpMin());
    small_moved = block_reduce<kSpineThreads>(small_moved, sh, OpAdd());
    if (threadIdx.x == 0) {
        const uint64_t tail = arena_bytes - hdr->max_live_end;
        // holes below live blocks come first in address order; the tail last
        if (min_fit == kNone && tail && tail >= fit_need) min_fit = hdr->max_live_end;
        hdr->fit_offset = min_fit;
        hdr->largest_hole = umax64(max_gap, tail);
        hdr->hole_count = gaps + (tail ? 1 : 0);
        hdr->moved_blocks = moved;
        hdr->moved_bytes = moved_bytes;
        hdr->small_moved = small_moved;
        hdr->min_live_size = min_size;
        hdr->move_begin = min_dst;
        // plan fields: a statistics-only pass leaves an existing plan intact
        if (outputs) {
            hdr->epoch = epoch;
            hdr->ticket = 0;
            hdr->status = 0;
            hdr->late_tiles = 0;
            hdr->waited_tiles = 0;
            hdr->polls = 0;
        }
    }
}

__global__ __launch_bounds__(kSpineThreads) void k_scan_finish(const StatPart *spart, uint64_t nb,
                                                               uint64_t arena_bytes, WsHeader *hdr,
                                                               int outputs, uint64_t epoch,
                                                               uint64_t fit_need) {
    scan_finish(spart, nb, arena_bytes, hdr, outputs, epoch, fit_need);
}

// ---------------------------------------------------------------------------
// Tiles.  A run is a maximal sequence of moved live blocks; its destinations
// are contiguous (packed inside one segment).  Its tiles are the pieces of it
// inside each tile-size window: one starts at the run's first byte, and one at
// every multiple of T inside the run.

__device__ inline bool moved_at(const LiveView &lv, uint64_t k) { return lv.src[k] != lv.dst[k]; }

// Tiles starting inside live block k (0 if k did not move).
__device__ inline uint64_t tiles_in_block(const LiveView &lv, uint64_t k, uint64_t T) {
    if (!moved_at(lv, k)) return 0;
    const bool start = (k == 0) || !moved_at(lv, k - 1);
    const uint64_t a = lv.dst[k], b = a + lv.size[k];
    const uint64_t mult = (b + T - 1) / T - (a + T - 1) / T;  // multiples of T in [a, b)
    return mult + ((start && (a & (T - 1))) ? 1 : 0);
}

// Whole windows [cT, cT + T) inside moved block k: each is one tile holding
// that block alone (the mover's straight-line case).
__device__ inline uint64_t whole_in_block(const LiveView &lv, uint64_t k, uint64_t T) {
    if (!moved_at(lv, k)) return 0;
    const uint64_t a = lv.dst[k], b = a + lv.size[k];
    const uint64_t lo = (a + T - 1) / T, hi = b / T;
    return hi > lo ? hi - lo : 0;
}

// Pass 5: per-workgroup tile counts (and whole-window counts) over the live
// blocks, for both tile-size candidates (tpart[blk], tpart[kMaxScanParts +
// blk]); workgroup blk covers live blocks [blk * chunk, (blk + 1) * chunk).
__device__ void tcount_partial(LiveView lv, const WsHeader *hdr, TileChoice tc, uint64_t *tpart,
                               uint64_t *twhole, uint64_t blk, uint64_t chunk) {
    __shared__ uint64_t sh[kScanThreads / 64];
    if (plan_dead(hdr)) return;
    const uint64_t m = hdr->live_blocks;
    const uint64_t end = umin64((blk + 1) * chunk, m);
    uint64_t ca = 0, wa = 0, cb = 0, wb = 0;
    for (uint64_t k0 = blk * chunk + (uint64_t)threadIdx.x * kScanItems; k0 < end;
         k0 += kScanTile) {
#pragma unroll
        for (uint32_t j = 0; j < kScanItems; ++j) {
            if (k0 + j < end) {
                ca += tiles_in_block(lv, k0 + j, tc.a);
                wa += whole_in_block(lv, k0 + j, tc.a);
                cb += tiles_in_block(lv, k0 + j, tc.b);
                wb += whole_in_block(lv, k0 + j, tc.b);
            }
        }
    }
    ca = block_reduce<kScanThreads>(ca, sh, OpAdd());
    wa = block_reduce<kScanThreads>(wa, sh, OpAdd());
    cb = block_reduce<kScanThreads>(cb, sh, OpAdd());
    wb = block_reduce<kScanThreads>(wb, sh, OpAdd());
    if (threadIdx.x == 0) {
        tpart[blk] = ca;
        twhole[blk] = wa;
        tpart[kMaxScanParts + blk] = cb;
        twhole[kMaxScanParts + blk] = wb;
    }
}

// The remap's bucket index: ridx[b] = number of live blocks whose old offset
// is below b << w, for b in [0, nb]; one lane per entry, a binary search over
// the packed old offsets (workgroup blk covers entries [256 blk, ...)).  A
// failed plan leaves it alone.
__device__ void remap_index_part(const uint64_t *__restrict__ live_src, const WsHeader *hdr,
                                 uint32_t w, uint64_t nb, uint32_t *ridx, uint64_t blk) {
    const uint64_t b = blk * kScanThreads + threadIdx.x;
    if (b > nb || plan_dead(hdr)) return;
    const uint64_t m = hdr->live_blocks;
    const uint64_t x = b << w;
    uint64_t lo = 0, len = m;  // first k with src[k] >= x
    while (len > 0) {
        const uint64_t half = len >> 1;
        if (live_src[lo + half] < x) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    ridx[b] = (uint32_t)lo;
}

// After a plan's scan, three jobs that read only what the scan wrote and
// write disjoint outputs, in one launch (two dependent launches fewer):
// workgroups [0, gnb) count tiles (pass 5), the next rblocks build the
// remap index, and the last one reduces the statistics (pass 4).
struct AfterScan {
    LiveView lv;
    TileChoice tiles;
    uint64_t *tpart, *twhole;
    uint64_t gnb;
    uint64_t chunk;     // live blocks per counting workgroup
    uint32_t *ridx;
    uint32_t rw;        // remap bucket width (log2 bytes)
    uint64_t rnb;       // remap buckets
    uint64_t rblocks;   // workgroups building the index
    const StatPart *spart;
    uint64_t nb;        // scan workgroups
    uint64_t arena_bytes;
    int outputs;
    uint64_t epoch;
    uint64_t fit_need;
};
static_assert(kSpineThreads == kScanThreads, "the finish runs as one workgroup of the fused launch");
__global__ __launch_bounds__(kScanThreads) void k_after_scan(AfterScan a, WsHeader *hdr) {
    const uint64_t blk = blockIdx.x;
    if (blk < a.gnb) {
        tcount_partial(a.lv, hdr, a.tiles, a.tpart, a.twhole, blk, a.chunk);
    } else if (blk < a.gnb + a.rblocks) {
        remap_index_part(a.lv.src, hdr, a.rw, a.rnb, a.ridx, blk - a.gnb);
    } else {
        scan_finish(a.spart, a.nb, a.arena_bytes, hdr, a.outputs, a.epoch, a.fit_need);
    }
}

// Pass 6 (one workgroup): the tile size, then the exclusive scan of its
// counts; n_tiles.  With two candidates the larger is taken when most moved
// bytes shift by less than kAutoSmallShift and enough bytes move -- or when
// the smaller's tiles would not fit the workspace and the larger's do.
__global__ __launch_bounds__(kSpineThreads) void k_tcount_spine(const uint64_t *tpart,
                                                                const uint64_t *twhole,
                                                                uint64_t *tprefix, uint64_t nb,
                                                                WsHeader *hdr, TileChoice tc,
                                                                uint64_t max_tiles) {
    __shared__ uint64_t sh[kSpineThreads / 64];
    if (plan_dead(hdr)) return;
    uint64_t na = 0, nbt = 0;
    for (uint64_t j = threadIdx.x; j < nb; j += kSpineThreads) {
        na += tpart[j];
        nbt += tpart[kMaxScanParts + j];
    }
    na = block_reduce<kSpineThreads>(na, sh, OpAdd());
    nbt = block_reduce<kSpineThreads>(nbt, sh, OpAdd());
    const uint64_t moved = hdr->moved_bytes;
    bool pick_b = tc.a != tc.b && hdr->small_moved * 2 > moved && moved >= kAutoMinMoved;
    if (tc.a != tc.b && (pick_b ? nbt : na) > max_tiles && (pick_b ? na : nbt) <= max_tiles)
        pick_b = !pick_b;
    const uint64_t off = pick_b ? kMaxScanParts : 0;
    uint64_t carry = 0, whole = 0;
    for (uint64_t j = threadIdx.x; j < nb; j += kSpineThreads) whole += twhole[off + j];
    whole = block_reduce<kSpineThreads>(whole, sh, OpAdd());
    for (uint64_t base = 0; base < nb; base += kSpineThreads) {
        const uint64_t j = base + threadIdx.x;
        const uint64_t x = j < nb ? tpart[off + j] : 0;
        uint64_t total;
        const uint64_t ex = block_excl_sum<kSpineThreads>(x, total, sh);
        if (j < nb) tprefix[j] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) {
        hdr->n_tiles = carry;
        hdr->whole_tiles = whole;
        hdr->tile_bytes = pick_b ? tc.b : tc.a;
    }
}

// Pass 7: each live block's first tile index (a block with no tile gets the
// same index as the next block that has one, so tile t belongs to the last
// block whose first tile index is <= t).
__global__ __launch_bounds__(kScanThreads) void k_tcount_down(LiveView lv, const WsHeader *hdr,
                                                              const uint64_t *tprefix,
                                                              uint32_t *tile_base, uint64_t chunk) {
    __shared__ uint64_t sh[kScanThreads / 64];
    if (plan_dead(hdr)) return;
    const uint64_t m = hdr->live_blocks;
    const uint64_t T = hdr->tile_bytes;
    const uint64_t base = (uint64_t)blockIdx.x * chunk;
    const uint64_t end = umin64(base + chunk, m);
    uint64_t carry = tprefix[blockIdx.x];
    for (uint64_t s0 = base; s0 < end; s0 += kScanTile) {
        const uint64_t k0 = s0 + (uint64_t)threadIdx.x * kScanItems;
        uint64_t c[kScanItems];
        uint64_t sum = 0;
#pragma unroll
        for (uint32_t j = 0; j < kScanItems; ++j) {
            c[j] = (k0 + j < end) ? tiles_in_block(lv, k0 + j, T) : 0;
            sum += c[j];
        }
        uint64_t total;
        uint64_t run = carry + block_excl_sum<kScanThreads>(sum, total, sh);
        carry += total;
#pragma unroll
        for (uint32_t j = 0; j < kScanItems; ++j) {
            if (k0 + j < end) tile_base[k0 + j] = (uint32_t)run;
            run += c[j];
        }
    }
}

// Largest k in [lo, hi) with a[k] <= x, or lo - 1 if none.
template <typename T>
__device__ inline int64_t last_le(const T *a, int64_t lo, int64_t hi, uint64_t x) {
    int64_t l = lo, h = hi;  // first index with a[k] > x in [lo, hi)
    while (l < h) {
        const int64_t mid = l + ((h - l) >> 1);
        if ((uint64_t)a[mid] <= x) l = mid + 1;
        else h = mid;
    }
    return l - 1;
}

// Pass 8: one lane per tile writes its start and its first block.
__global__ __launch_bounds__(256) void k_tile_starts(LiveView lv, const uint32_t *tile_base,
                                                     const WsHeader *hdr, uint64_t max_tiles,
                                                     uint64_t *tile_start, uint32_t *tile_first) {
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (plan_dead(hdr) || hdr->n_tiles > max_tiles) return;  // plan fails
    const uint64_t n_tiles = hdr->n_tiles, m = hdr->live_blocks, T = hdr->tile_bytes;
    if (t >= n_tiles) return;
    const int64_t k = last_le(tile_base, 0, (int64_t)m, t);
    const uint64_t j = t - tile_base[k];
    const uint64_t a = lv.dst[k];
    const bool start = (k == 0) || !moved_at(lv, (uint64_t)k - 1);
    const uint64_t lead = (start && (a & (T - 1))) ? 1 : 0;
    const uint64_t first_mult = (a + T - 1) & ~(T - 1);
    tile_start[t] = (j < lead) ? a : first_mult + (j - lead) * T;
    tile_first[t] = (uint32_t)k;
}

// The tile holding destination byte q of moved block b (tiles cut each run
// at its start and at every multiple of T).
__device__ inline uint64_t tile_of(const LiveView &lv, const uint32_t *tile_base, uint64_t b,
                                   uint64_t q, uint64_t T) {
    const uint64_t a = lv.dst[b];
    const uint64_t A = (a + T - 1) & ~(T - 1);
    const bool start = (b == 0) || !moved_at(lv, b - 1);
    const uint64_t lead = (start && (a & (T - 1))) ? 1 : 0;
    if (q >= A) return tile_base[b] + lead + (q - A) / T;
    // q lies in the window block b starts in: block b's own first tile if it
    // starts a run there, else the tile that began earlier in the run
    return lead ? tile_base[b] : tile_base[b] - 1;
}

// Pass 9: one lane per tile.  [t0, t1) = the run's bytes from the tile start
// up to the next tile start, the window end or the run end.  A tile may write
// only once every tile whose sources overlap [t0, t1) has read them.  Sources
// rise strictly with destinations (src = dst + shift, shifts never negative,
// order kept), so the destinations whose sources lie in [t0, t1) are at most
// t1 - t0 consecutive live bytes, all at or below [t0, t1): their tiles are a
// short range ending at or before this one.
__global__ __launch_bounds__(256) void k_tiles(LiveView lv, const uint64_t *tile_start,
                                               const uint32_t *tile_first,
                                               const uint32_t *tile_base, const WsHeader *hdr,
                                               uint64_t max_tiles,
                                               const uint32_t *ridx, uint32_t w, TileRec *tiles,
                                               uint32_t *flags) {
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (plan_dead(hdr) || hdr->n_tiles > max_tiles) return;  // plan fails
    const uint64_t n_tiles = hdr->n_tiles, m = hdr->live_blocks, T = hdr->tile_bytes;
    if (t >= n_tiles) return;
    const uint64_t t0 = tile_start[t];
    uint64_t bound = (t0 & ~(T - 1)) + T;
    if (t + 1 < n_tiles) bound = umin64(bound, tile_start[t + 1]);
    const uint64_t first = tile_first[t];
    // last block of the run inside [t0, bound): blocks after first that start
    // below bound and moved form a prefix -- gallop, then bisect
    uint64_t last = first, stride = 1;
    while (last + stride < m && lv.dst[last + stride] < bound && moved_at(lv, last + stride)) {
        last += stride;
        stride <<= 1;
    }
    for (; stride > 0; stride >>= 1)
        if (last + stride < m && lv.dst[last + stride] < bound && moved_at(lv, last + stride))
            last += stride;
    const uint64_t t1 = umin64(bound, lv.dst[last] + lv.size[last]);
    // sources overlapping [t0, t1): first block whose source ends above t0.
    // The remap index narrows it to the blocks starting in t0's bucket and
    // the one before them: an earlier block ends before the bucket starts,
    // and the first block of the next bucket already ends above t0.
    const uint64_t bk = t0 >> w;
    int64_t lo = ridx[bk] ? (int64_t)ridx[bk] - 1 : 0, hi = (int64_t)ridx[bk + 1];
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (lv.src[mid] + lv.size[mid] <= t0) lo = mid + 1;
        else hi = mid;
    }
    uint32_t dep_lo = 1, dep_hi = 0;  // empty
    if (lo < (int64_t)m && lv.src[lo] < t1 && t > 0) {
        const uint64_t j = (uint64_t)lo;
        const uint64_t q_lo = lv.dst[j] + (t0 > lv.src[j] ? t0 - lv.src[j] : 0);
        // ... and the last block whose source starts below t1 (gallop from j)
        uint64_t c = j;
        stride = 1;
        while (c + stride < m && lv.src[c + stride] < t1) {
            c += stride;
            stride <<= 1;
        }
        for (; stride > 0; stride >>= 1)
            if (c + stride < m && lv.src[c + stride] < t1) c += stride;
        const uint64_t q_hi = lv.dst[c] + umin64(lv.size[c], t1 - lv.src[c]) - 1;
        const uint64_t u_lo = tile_of(lv, tile_base, j, q_lo, T);
        uint64_t u_hi = tile_of(lv, tile_base, c, q_hi, T);
        if (u_hi > t - 1) u_hi = t - 1;
        if (u_lo <= u_hi) {
            dep_lo = (uint32_t)u_lo;
            dep_hi = (uint32_t)u_hi;
        }
    }
    tiles[t] = TileRec{t0, t1, lv.src[first] - lv.dst[first], (uint32_t)first, (uint32_t)last,
                       dep_lo, dep_hi, 0};
    flags[t] = 0u;
}

__global__ void k_commit(LiveView lv, uint64_t m, uint64_t *off_out, uint64_t *size_out,
                         uint8_t *live_out, uint8_t *pinned_out) {
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < m;
         k += (uint64_t)gridDim.x * blockDim.x) {
        if (off_out) off_out[k] = lv.dst[k];
        if (size_out) size_out[k] = lv.size[k];
        if (live_out) live_out[k] = 1;
        if (pinned_out) pinned_out[k] = lv.pin[k];
    }
}

// ---------------------------------------------------------------------------
// Targeted compaction.  Page: "Ascend 910C cluster tuning", section "Periodic
// compaction with Ascend C": compaction pauses what it touches and is kept for
// stopping the damage, and the failure it answers is one request larger than
// any free block.  Number the holes by the live block just above them (hole q
// lies below live block q; hole m is the tail), and let
//   B_q = hole bytes below live block q's start  (B_m = free total)
//   Z_q = live bytes below live block q          (Z_m = live total)
// both non-decreasing.  The window of holes k..l (k <= l) holds live blocks
// k..l-1; packed down to its start they free B_l - B_{k-1} bytes in one piece
// (B_{-1} = 0) and move Z_l - Z_k bytes.  It may hold no pinned block.  For a
// last hole l the cheapest window is the one with the largest k that still
// frees the request, found by binary search over B; the best over all l --
// fewest moved bytes, then lowest k -- is the window.

__device__ inline uint64_t holes_below(const uint64_t *src, const uint64_t *z, uint64_t q,
                                       uint64_t m, uint64_t free_total) {
    return q < m ? src[q] - z[q] : free_total;
}

__device__ inline bool sel_better(uint64_t c1, uint64_t k1, uint64_t c2, uint64_t k2) {
    return c1 < c2 || (c1 == c2 && k1 < k2);
}

// Workgroup arg-min of (cost, k) carrying l, through LDS (NT threads).
template <int NT>
__device__ inline void sel_reduce(uint64_t &c, uint64_t &k, uint64_t &l, uint64_t *sh) {
    constexpr int NW = NT / 64;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint64_t c2 = __shfl_xor(c, d, 64), k2 = __shfl_xor(k, d, 64),
                       l2 = __shfl_xor(l, d, 64);
        if (sel_better(c2, k2, c, k)) {
            c = c2;
            k = k2;
            l = l2;
        }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sh[3 * w] = c;
        sh[3 * w + 1] = k;
        sh[3 * w + 2] = l;
    }
    __syncthreads();
    c = sh[0];
    k = sh[1];
    l = sh[2];
#pragma unroll
    for (int j = 1; j < NW; ++j) {
        if (sel_better(sh[3 * j], sh[3 * j + 1], c, k)) {
            c = sh[3 * j];
            k = sh[3 * j + 1];
            l = sh[3 * j + 2];
        }
    }
    __syncthreads();
}

// One lane per candidate last hole l in [0, m].
__global__ __launch_bounds__(kSelThreads) void k_select(const uint64_t *src, const uint64_t *z,
                                                        const uint32_t *pc, const WsHeader *hdr,
                                                        uint64_t arena_bytes, uint64_t request,
                                                        SelPart *sp) {
    __shared__ uint64_t sh[3 * (kSelThreads / 64)];
    if (hdr->bad_key != kNone) return;
    const uint64_t m = hdr->live_blocks, lt = hdr->live_bytes, np = hdr->pinned_blocks;
    const uint64_t free_total = arena_bytes - lt;
    const uint64_t l = (uint64_t)blockIdx.x * kSelThreads + threadIdx.x;
    uint64_t cost = kNone, kk = kNone, ll = kNone;
    if (l <= m) {
        const uint64_t bl = holes_below(src, z, l, m, free_total);
        if (bl >= request) {
            const uint64_t x = bl - request;
            // first q in [0, l) with B_q > x; then k = q
            uint64_t lo = 0, len = l;
            while (len > 0) {
                const uint64_t half = len >> 1, q = lo + half;
                if (src[q] - z[q] <= x) {
                    lo = q + 1;
                    len -= half + 1;
                } else {
                    len = half;
                }
            }
            const uint64_t k = lo;
            const uint64_t pl = l < m ? pc[l] : np, pk = k < m ? pc[k] : np;
            if (pl == pk) {  // no pinned block among k..l-1
                cost = (l < m ? z[l] : lt) - (k < m ? z[k] : lt);
                kk = k;
                ll = l;
            }
        }
    }
    sel_reduce<kSelThreads>(cost, kk, ll, sh);
    if (threadIdx.x == 0) sp[blockIdx.x] = SelPart{cost, kk, ll, 0};
}

// One workgroup: the best window over all candidates, as bytes.
__global__ __launch_bounds__(kSpineThreads) void k_select_finish(const SelPart *sp, uint64_t nb,
                                                                 const uint64_t *src,
                                                                 const uint64_t *size,
                                                                 const uint64_t *z,
                                                                 uint64_t arena_bytes,
                                                                 WsHeader *hdr) {
    __shared__ uint64_t sh[3 * (kSpineThreads / 64)];
    if (hdr->bad_key != kNone) return;
    uint64_t c = kNone, k = kNone, l = kNone;
    for (uint64_t j = threadIdx.x; j < nb; j += kSpineThreads) {
        const SelPart q = sp[j];
        if (sel_better(q.cost, q.k, c, k)) {
            c = q.cost;
            k = q.k;
            l = q.l;
        }
    }
    sel_reduce<kSpineThreads>(c, k, l, sh);
    if (threadIdx.x != 0) return;
    if (c == kNone) {
        hdr->win_state = kWinNoFit;
        hdr->win_begin = hdr->win_end = hdr->win_hole = hdr->win_moved = 0;
        return;
    }
    const uint64_t m = hdr->live_blocks;
    const uint64_t free_total = arena_bytes - hdr->live_bytes;
    const uint64_t below = k ? holes_below(src, z, k - 1, m, free_total) : 0;
    hdr->win_begin = k ? src[k - 1] + size[k - 1] : 0;
    hdr->win_end = l < m ? src[l] : arena_bytes;
    hdr->win_hole = holes_below(src, z, l, m, free_total) - below;
    hdr->win_moved = c;
    hdr->win_state = kWinFound;
}

}  // namespace

namespace {

// Scan passes, then (kOutNew) the tile passes.  win: the targeted plan's
// window in the header, or null.
hipError_t queue_scan(const TableView &t, uint64_t arena_bytes, uint8_t *ws, const WsLayout &L,
                uint64_t *new_offset, int outputs, const uint64_t *win, TileChoice tiles,
                uint64_t epoch, uint64_t fit_need, hipStream_t s) {
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    ScanPart *part = reinterpret_cast<ScanPart *>(ws + L.part);
    ScanPart *prefix = reinterpret_cast<ScanPart *>(ws + L.prefix);
    StatPart *spart = reinterpret_cast<StatPart *>(ws + L.spart);
    LiveOut lo{reinterpret_cast<uint64_t *>(ws + L.live_dst),
               reinterpret_cast<uint64_t *>(ws + L.live_src),
               reinterpret_cast<uint64_t *>(ws + L.live_size),
               reinterpret_cast<uint8_t *>(ws + L.live_pin),
               reinterpret_cast<uint64_t *>(ws + L.live_z),
               reinterpret_cast<uint32_t *>(ws + L.live_pc),
               nullptr, nullptr, nullptr, nullptr, 0};
    if (remap_ent(arena_bytes, t.n)) {
        lo.ent = reinterpret_cast<RemapEnt *>(ws + L.live_rec);
        lo.key_mask = (1ull << remap_shift(arena_bytes, t.n)) - 1;
    } else if (remap_rec32(arena_bytes)) {
        lo.rec32 = reinterpret_cast<LiveRec32 *>(ws + L.live_rec);
    } else {
        lo.rec = reinterpret_cast<LiveRec *>(ws + L.live_rec);
    }
    if (!lo.ent && remap_keys32(arena_bytes, t.n)) {
        lo.key = reinterpret_cast<uint32_t *>(ws + L.live_key);
        lo.key_mask = (1ull << remap_shift(arena_bytes, t.n)) - 1;
    }
    const uint64_t nb = L.n_scan_blocks;
    if (nb) {
        hipLaunchKernelGGL(k_scan_partials, dim3((uint32_t)nb), dim3(kScanThreads), 0, s, t,
                           arena_bytes, win, (uint64_t)L.scan_chunk, part);
        AC_TRY(hipGetLastError());
    }
    hipLaunchKernelGGL(k_scan_spine, dim3(1), dim3(kSpineThreads), 0, s, part, prefix, nb, hdr,
                       win ? 0 : 1);
    AC_TRY(hipGetLastError());
    if (nb) {
        hipLaunchKernelGGL(k_scan_down, dim3((uint32_t)nb), dim3(kScanThreads), 0, s, t, win,
                           prefix, hdr, new_offset, lo, spart, outputs, fit_need,
                           (uint64_t)L.scan_chunk);
        AC_TRY(hipGetLastError());
    }
    if (!(outputs & kOutNew)) {
        hipLaunchKernelGGL(k_scan_finish, dim3(1), dim3(kSpineThreads), 0, s, spart, nb,
                           arena_bytes, hdr, outputs, epoch, fit_need);
        AC_TRY(hipGetLastError());
    }
    if (outputs & kOutNew) {
        const LiveView lv = live_view(ws, L);
        uint64_t *tpart = reinterpret_cast<uint64_t *>(ws + L.tpart);
        uint64_t *tprefix = reinterpret_cast<uint64_t *>(ws + L.tprefix);
        uint64_t *twhole = reinterpret_cast<uint64_t *>(ws + L.twhole);
        uint32_t *tile_base = reinterpret_cast<uint32_t *>(ws + L.tile_base);
        const uint64_t gnb = nb ? nb : 1;  // live blocks <= entries
        // tile counts, the remap's bucket index (the tile records use it
        // too) and the statistics finish, in one launch
        uint32_t *ridx = reinterpret_cast<uint32_t *>(ws + L.ridx);
        AfterScan as{};
        as.lv = lv;
        as.tiles = tiles;
        as.tpart = tpart;
        as.twhole = twhole;
        as.gnb = gnb;
        as.chunk = L.scan_chunk;
        as.ridx = ridx;
        as.rw = remap_shift(arena_bytes, t.n);
        as.rnb = remap_buckets(arena_bytes, t.n);
        as.rblocks = (as.rnb + 1 + kScanThreads - 1) / kScanThreads;
        as.spart = spart;
        as.nb = nb;
        as.arena_bytes = arena_bytes;
        as.outputs = outputs;
        as.epoch = epoch;
        as.fit_need = fit_need;
        hipLaunchKernelGGL(k_after_scan, dim3((uint32_t)(gnb + as.rblocks + 1)),
                           dim3(kScanThreads), 0, s, as, hdr);
        AC_TRY(hipGetLastError());
        hipLaunchKernelGGL(k_tcount_spine, dim3(1), dim3(kSpineThreads), 0, s, tpart, twhole,
                           tprefix, gnb, hdr, tiles, (uint64_t)L.max_tiles);
        AC_TRY(hipGetLastError());
        hipLaunchKernelGGL(k_tcount_down, dim3((uint32_t)gnb), dim3(kScanThreads), 0, s, lv, hdr,
                           tprefix, tile_base, (uint64_t)L.scan_chunk);
        AC_TRY(hipGetLastError());
        // tile starts and records: a grid for the whole capacity, each lane
        // checks the device-side tile count (no host round trip)
        uint64_t *tile_start = reinterpret_cast<uint64_t *>(ws + L.tile_start);
        uint32_t *tile_first = reinterpret_cast<uint32_t *>(ws + L.tile_first);
        TileRec *trec = reinterpret_cast<TileRec *>(ws + L.tiles);
        uint32_t *flags = reinterpret_cast<uint32_t *>(ws + L.flags);
        const uint64_t grid = (L.max_tiles + 255) / 256;
        if (grid) {
            hipLaunchKernelGGL(k_tile_starts, dim3((uint32_t)grid), dim3(256), 0, s, lv, tile_base,
                               hdr, L.max_tiles, tile_start, tile_first);
            AC_TRY(hipGetLastError());
            hipLaunchKernelGGL(k_tiles, dim3((uint32_t)grid), dim3(256), 0, s, lv, tile_start,
                               tile_first, tile_base, hdr, L.max_tiles,
                               ridx, remap_shift(arena_bytes, t.n), trec, flags);
            AC_TRY(hipGetLastError());
        }
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_scan(const TableView &t, uint64_t arena_bytes, uint8_t *ws, const WsLayout &L,
                       uint64_t *new_offset, int outputs, TileChoice tiles, uint64_t epoch,
                       uint64_t fit_need, hipStream_t s) {
    return queue_scan(t, arena_bytes, ws, L, new_offset, outputs, nullptr, tiles, epoch,
                      fit_need, s);
}

hipError_t launch_targeted(const TableView &t, uint64_t arena_bytes, uint64_t request,
                           uint8_t *ws, const WsLayout &L, uint64_t *new_offset,
                           TileChoice tiles, uint64_t epoch, hipStream_t s) {
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    const uint64_t *src = reinterpret_cast<const uint64_t *>(ws + L.live_src);
    const uint64_t *size = reinterpret_cast<const uint64_t *>(ws + L.live_size);
    const uint64_t *z = reinterpret_cast<const uint64_t *>(ws + L.live_z);
    const uint32_t *pc = reinterpret_cast<const uint32_t *>(ws + L.live_pc);
    SelPart *sp = reinterpret_cast<SelPart *>(ws + L.selpart);
    AC_TRY(queue_scan(t, arena_bytes, ws, L, nullptr, kOutSelect, nullptr, tiles, epoch,
                      kNone, s));
    // candidates: every last hole l in [0, m], m <= n
    hipLaunchKernelGGL(k_select, dim3((uint32_t)L.n_sel_blocks), dim3(kSelThreads), 0, s, src, z,
                       pc, hdr, arena_bytes, request, sp);
    AC_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_select_finish, dim3(1), dim3(kSpineThreads), 0, s, sp, L.n_sel_blocks,
                       src, size, z, arena_bytes, hdr);
    AC_TRY(hipGetLastError());
    return queue_scan(t, arena_bytes, ws, L, new_offset, kOutNew, &hdr->win_begin, tiles,
                      epoch, kNone, s);
}

hipError_t launch_commit(const uint8_t *ws, const WsLayout &L, uint64_t live_blocks,
                         uint64_t *off_out, uint64_t *size_out, uint8_t *live_out,
                         uint8_t *pinned_out, hipStream_t s) {
    if (live_blocks == 0) return hipSuccess;
    uint64_t grid = (live_blocks + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_commit, dim3((uint32_t)grid), dim3(256), 0, s, live_view(ws, L),
                       live_blocks, off_out, size_out, live_out, pinned_out);
    return hipGetLastError();
}

}  // namespace ac

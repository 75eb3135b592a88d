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
// A plan's passes (n up to 2^32 entries), each a wide launch with no
// one-workgroup pass between them: every workgroup of a pass scans the (at
// most 1,024) per-workgroup results of the pass before it for its own
// prefix, since each dependent launch costs several microseconds of
// dispatch.
//   1. per-workgroup aggregates (and the first bad entry);
//   2. each workgroup's prefix, then its entries: new offsets, the packed
//      live-block arrays (new and old offset, size, pinned flag, the remap's
//      records), hole and move statistics, and the tiles its moved blocks
//      start, counted for both candidate tile sizes; workgroup 0 writes the
//      table's totals;
//   3. each workgroup picks the tile size from the totals, the same way, and
//      gives each of its live blocks its first tile index; one more
//      workgroup finishes the header (statistics, tile count and size, the
//      mover's fields); further workgroups build the remap's bucket index
//      over old offsets (it also narrows the tiles' source searches);
//   4. one lane per tile: its start, range, blocks and dependencies.
// The whole sequence is queued at once; the host reads the header back only
// at the end.  A statistics pass alone is one launch of its own
// (k_stats_one), which needs no prefix.
#include "stats_one.h"

namespace ac {
namespace {

// Nothing more to plan: the table is invalid, or no window fits the request.
__device__ inline bool plan_dead(const WsHeader *hdr) {
    const uint64_t bad = hdr->bad_key, win = hdr->win_state;  // both loads, then the tests
    return (bad != kNone) | (win == kWinNoFit);
}

// Pass 1: per-workgroup aggregate and first bad key.  Workgroup g takes the
// entries [g * chunk, (g + 1) * chunk), kScanTile at a time.
__global__ __launch_bounds__(kScanThreads) void k_scan_partials(TableView t, uint64_t arena_bytes,
                                                                const uint64_t *win,
                                                                uint64_t chunk, ScanPart *part) {
    __shared__ Agg sh[kExclSlots<kScanThreads>];
    __shared__ uint64_t shr[kScanThreads / 64];
    const uint64_t n = t.n;
    const Window w = window_of(win);
    const uint64_t base = (uint64_t)blockIdx.x * chunk;
    const uint64_t end = umin64(base + chunk, n);
    Agg acc = agg_zero();
    uint64_t bad = kNone;
    for (uint64_t s0 = base; s0 < end; s0 += kScanTile) {
        const uint64_t i0 = s0 + (uint64_t)threadIdx.x * kScanItems;
        Agg a = agg_zero();
        uint64_t prev_end = 0;
        if (i0 > 0 && i0 < n) prev_end = t.off[i0 - 1] + t.size[i0 - 1];
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            if (i < n) {
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

// Every pass after the aggregates takes what it needs of them itself: each
// workgroup scans the (at most kMaxScanParts) aggregates for its own prefix
// and the table's totals -- a few microseconds of L2-resident work in every
// workgroup, in place of a one-workgroup launch and the gap in front of it.
// before: aggregates of the parts below g; total: of all; bad: the smallest
// bad-entry key.  s_before: an LDS slot for the broadcast.
__device__ void parts_prefix(const ScanPart *part, uint64_t nb, uint64_t g, Agg *sh,
                             uint64_t *shr, Agg *s_before, Agg &before, Agg &total,
                             uint64_t &bad) {
    if (nb <= 64) {
        // few aggregates: the first wave scans them, one a lane, and hands
        // out the prefix, the total and the first bad key through LDS (two
        // barriers where the general path below takes five)
        if (threadIdx.x < 64) {
            const uint32_t j = threadIdx.x;
            Agg x = agg_zero();
            uint64_t b = kNone;
            if (j < nb) {
                x = part[j].a;
                b = part[j].bad_key;
            }
            const Agg inc = agg_incl_scan(x);
            const Agg ex = agg_shift_up(inc);
            b = wave_reduce(b, umin64);
            if (j == g) *s_before = ex;
            if (j == 63) sh[0] = inc;  // lanes past nb add the identity: the total
            if (j == 0) shr[0] = b;
        }
        __syncthreads();
        before = wave_uniform(*s_before);
        total = wave_uniform(sh[0]);
        bad = wave_uniform(shr[0]);
        __syncthreads();  // sh and shr are the caller's next scan's
        return;
    }
    constexpr uint32_t kPer = kMaxScanParts / kScanThreads;
    const uint64_t j0 = (uint64_t)threadIdx.x * kPer;
    Agg loc = agg_zero(), upto = agg_zero();
    uint64_t b = kNone;
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        const uint64_t j = j0 + k;
        if (j == g) upto = loc;
        if (j < nb) {
            loc = combine(loc, part[j].a);
            b = umin64(b, part[j].bad_key);
        }
    }
    const Agg ex = block_excl<kScanThreads>(loc, total, sh);
    if (g >= j0 && g < j0 + kPer) *s_before = combine(ex, upto);
    bad = block_reduce<kScanThreads>(b, shr, OpMin());  // (its barriers publish s_before)
    before = wave_uniform(*s_before);
}

// The same for sums of u64 (tile counts): the sum below g and the total.
// v: this thread's values x[threadIdx.x * kPartsPer + k] (0 past the end),
// loaded by the caller.
constexpr uint32_t kPartsPer = kMaxScanParts / kScanThreads;
__device__ void sums_prefix(const uint64_t (&v)[kPartsPer], uint64_t g, uint64_t *sh,
                            uint64_t *s_before, uint64_t &before, uint64_t &total) {
    constexpr uint32_t kPer = kPartsPer;
    const uint64_t j0 = (uint64_t)threadIdx.x * kPer;
    uint64_t loc = 0, upto = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        if (j0 + k == g) upto = loc;
        loc += v[k];
    }
    const uint64_t ex = block_excl_sum<kScanThreads>(loc, total, sh);
    if (g >= j0 && g < j0 + kPer) *s_before = ex + upto;
    __syncthreads();
    before = wave_uniform(*s_before);
    __syncthreads();
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

// Tiles a run of moved blocks starts in one live block: at the run's first
// byte (if not on a window boundary) and at every multiple of T inside it.
// a: new offset, s: size, start: the block opens a run.
// T is a power of two: x / T is a shift.
__device__ inline uint64_t div_tile(uint64_t x, uint64_t T) { return x >> __builtin_ctzll(T); }

__device__ inline uint64_t tiles_of(uint64_t a, uint64_t s, bool start, uint64_t T) {
    const uint64_t b = a + s;
    const uint64_t mult = div_tile(b + T - 1, T) - div_tile(a + T - 1, T);  // multiples of T in [a, b)
    return mult + ((start && (a & (T - 1))) ? 1 : 0);
}
// Whole windows [cT, cT + T) inside a moved block: each is one tile of that
// block alone.
__device__ inline uint64_t whole_of(uint64_t a, uint64_t s, uint64_t T) {
    const uint64_t lo = div_tile(a + T - 1, T), hi = div_tile(a + s, T);
    return hi > lo ? hi - lo : 0;
}

// The header's statistics from the reduced per-workgroup statistics q (the
// tail hole added), and the plan's mover fields reset.  max_end: the highest
// live end (the header's max_live_end).  One lane.
__device__ void stats_header(const StatPart &q, uint64_t arena_bytes, uint64_t max_end,
                             uint64_t fit_need, WsHeader *hdr) {
    const uint64_t tail = arena_bytes - max_end;
    uint64_t min_fit = q.min_fit;
    // holes below live blocks come first in address order; the tail last
    if (min_fit == kNone && tail && tail >= fit_need) min_fit = max_end;
    hdr->fit_offset = min_fit;
    hdr->largest_hole = umax64(q.max_gap, tail);
    hdr->hole_count = q.gaps + (tail ? 1 : 0);
    hdr->moved_blocks = q.moved_blocks;
    hdr->moved_bytes = q.moved_bytes;
    hdr->small_moved = q.small_moved;
    hdr->min_live_size = q.min_size;
    hdr->move_begin = q.min_moved_dst;
    hdr->ticket = 0;
    hdr->status = 0;
    hdr->late_tiles = 0;
    hdr->waited_tiles = 0;
    hdr->polls = 0;
}

// What a workgroup's entries add up to in the down-sweep: hole and move
// statistics, and the tiles its moved blocks start (and the whole windows
// they fill) for both candidate tile sizes.
struct DownAcc {
    uint64_t max_gap = 0, gaps = 0, moved = 0, moved_bytes = 0, min_dst = kNone,
             min_size = kNone, min_fit = kNone, small_moved = 0, ca = 0, wa = 0, cb = 0, wb = 0;
};

// One entry of the down-sweep: entry i (offset o, size s, live l, pinned p,
// stays f) after the scan state `run` of the entries before it.  Writes its
// new offset and, if live, its packed-array entries (at index run.cnt);
// adds to `acc`; leaves `run` past it.  OUT: the pass's outputs.
template <int OUT>
__device__ inline void down_item(uint64_t i, uint64_t o, uint64_t s, uint32_t l, uint32_t p,
                                 uint32_t f, Agg &run, uint64_t *new_offset, const LiveOut &lo,
                                 uint64_t fit_need, TileChoice tc, DownAcc &acc) {
    const uint64_t nw = f ? o : run.v;
    if ((OUT & kOutNew) && new_offset) new_offset[i] = nw;
    if (l) {
        if constexpr ((OUT & kOutNew) != 0) {
            lo.dst[run.cnt] = nw;
            lo.pin[run.cnt] = (uint8_t)p;
            if (lo.ent)
                lo.ent[run.cnt] = RemapEnt{(uint32_t)(o & lo.key_mask), (uint32_t)((o + s) >> 5),
                                           (uint32_t)((o - nw) >> 5), 0u};
            else if (lo.rec32)
                lo.rec32[run.cnt] = LiveRec32{(uint32_t)((o + s) >> 5), (uint32_t)((o - nw) >> 5)};
            else
                lo.rec[run.cnt] = LiveRec{o + s, o - nw};
            if (lo.key) lo.key[run.cnt] = (uint32_t)(o & lo.key_mask);
        }
        if constexpr ((OUT & (kOutNew | kOutSelect)) != 0) {
            lo.src[run.cnt] = o;
            lo.size[run.cnt] = s;
        }
        if constexpr ((OUT & kOutSelect) != 0) {
            lo.z[run.cnt] = run.lsum;
            lo.pc[run.cnt] = (uint32_t)run.pcnt;
        }
        const uint64_t gap = o - run.mx;
        if (gap) {
            acc.gaps += 1;
            acc.max_gap = umax64(acc.max_gap, gap);
            if (gap >= fit_need) acc.min_fit = umin64(acc.min_fit, run.mx);
        }
        if (o != nw) {
            acc.moved += 1;
            acc.moved_bytes += s;
            acc.min_dst = umin64(acc.min_dst, nw);
            if (o - nw < kAutoSmallShift) acc.small_moved += s;
            if constexpr ((OUT & kOutNew) != 0) {
                // the live block before this one moved: the run goes on
                const bool start = !(run.cnt > 0 && run.v != run.mx);
                acc.ca += tiles_of(nw, s, start, tc.a);
                acc.wa += whole_of(nw, s, tc.a);
                acc.cb += tiles_of(nw, s, start, tc.b);
                acc.wb += whole_of(nw, s, tc.b);
            }
        }
        acc.min_size = umin64(acc.min_size, s);
    }
    run = combine(run, element(o, s, l, p, f));
}

struct DownArgs {
    TableView t;
    const uint64_t *win;      // a targeted plan's window (in its header), or null
    const ScanPart *part;
    uint64_t nb;       // aggregates (0 for an empty table)
    uint64_t ngroups;  // workgroups of this pass: max(nb, 1)
    uint64_t chunk;
    WsHeader *hdr;
    uint64_t *new_offset;
    LiveOut lo;
    StatPart *spart;
    uint64_t *tpart, *twhole;  // tile counts per workgroup, both candidates (plans)
    uint64_t *lbase;           // live blocks below each workgroup's entries (plans; ngroups + 1)
    TileChoice tiles;
    uint64_t fit_need;
    uint64_t epoch;
    uint64_t arena_bytes;
};

// Pass 2: the workgroup's prefix (from the aggregates), then its entries in
// order: new offsets, the packed live arrays, hole and move statistics, and
// (plans) the tiles its moved blocks start, for both tile-size candidates.
// Workgroup 0 writes the table's totals and validity to the header.  An
// invalid table writes nothing else.  The block before a live entry moved
// iff the packed position after it differs from its end (a block that stays,
// pinned or held, resets the position to its own end).
// OUT: the pass's outputs (kOutNew: a plan; kOutSelect: a selection scan),
// fixed per instantiation so that each holds only its own code.
template <int OUT>
__global__ __launch_bounds__(kScanThreads) void k_scan_down(DownArgs d) {
    __shared__ Agg sh[kExclSlots<kScanThreads>];
    __shared__ uint64_t shr[kScanThreads / 64];
    __shared__ uint64_t s_red[kStatSlots<kScanThreads>];
    __shared__ Agg s_before;
    const TableView &t = d.t;
    const uint64_t g = blockIdx.x;
    const uint64_t n = t.n;
    const uint64_t base = g * d.chunk;
    const uint64_t end = umin64(base + d.chunk, n);
    uint64_t o[kScanItems], s[kScanItems];
    uint32_t l[kScanItems], p[kScanItems];
    const auto load = [&](uint64_t s0) {
        const uint64_t i0 = s0 + (uint64_t)threadIdx.x * kScanItems;
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            o[k] = 0;
            s[k] = 0;
            l[k] = 0;
            p[k] = 0;
            if (i < n) {
                o[k] = t.off[i];
                s[k] = t.size[i];
                l[k] = live_of(t, i) ? 1u : 0u;
                p[k] = pin_of(t, i) ? 1u : 0u;
            }
        }
    };
    // the first step's entries are requested before the prefix's aggregates,
    // so that the two loads overlap
    if (base < end) load(base);
    Agg before, total;
    uint64_t bad;
    parts_prefix(d.part, d.nb, g, sh, shr, &s_before, before, total, bad);
    const bool no_fit = d.win && d.hdr->win_state == kWinNoFit;  // set before this pass
    if (g == 0 && threadIdx.x == 0) {
        WsHeader *hdr = d.hdr;
        hdr->live_bytes = total.lsum;
        hdr->max_live_end = total.mx;
        hdr->live_blocks = total.cnt;
        hdr->pinned_blocks = total.pcnt;
        hdr->bad_key = bad;
        if (!d.win) hdr->win_state = kWinNone;
        // a plan (or a selection) overwrites the packed arrays: an older plan
        // in the workspace goes stale
        if (OUT && bad == kNone && !no_fit) hdr->epoch = d.epoch;
        if ((OUT & kOutNew) && bad == kNone && !no_fit) d.lbase[d.ngroups] = total.cnt;
    }
    if (bad != kNone || no_fit) return;  // invalid table or nothing to plan: write nothing
    const Window w = window_of(d.win);
    constexpr bool tiles = (OUT & kOutNew) != 0;
    if (tiles && threadIdx.x == 0) d.lbase[g] = before.cnt;
    Agg carry = before;
    DownAcc acc;
    for (uint64_t s0 = base; s0 < end; s0 += kScanTile) {
        if (s0 != base) load(s0);
        const uint64_t i0 = s0 + (uint64_t)threadIdx.x * kScanItems;
        uint32_t f[kScanItems];
        Agg a = agg_zero();
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            f[k] = 0;
            if (i < n) {
                f[k] = stays(o[k], l[k], p[k], w);
                a = combine(a, element(o[k], s[k], l[k], p[k], f[k]));
            }
        }
        Agg tot;
        const Agg ex = block_excl<kScanThreads>(a, tot, sh);
        Agg run = combine(carry, ex);
        carry = combine(carry, tot);
#pragma unroll
        for (uint32_t k = 0; k < kScanItems; ++k) {
            const uint64_t i = i0 + k;
            if (i < n)
                down_item<OUT>(i, o[k], s[k], l[k], p[k], f[k], run, d.new_offset, d.lo,
                               d.fit_need, d.tiles, acc);
        }
    }  // steps of the chunk
    StatPart q{acc.max_gap, acc.gaps, acc.moved, acc.moved_bytes, acc.min_dst, acc.min_size,
               acc.min_fit, acc.small_moved};
    uint64_t x[4] = {acc.ca, acc.wa, acc.cb, acc.wb};
    block_reduce_stats<kScanThreads>(q, x, s_red);
    if (threadIdx.x == 0) {
        d.spart[g] = q;
        if (tiles) {
            d.tpart[g] = x[0];
            d.twhole[g] = x[1];
            d.tpart[kMaxScanParts + g] = x[2];
            d.twhole[kMaxScanParts + g] = x[3];
        }
    }
}


__global__ void k_clear_u64(uint64_t *p) {
    if (threadIdx.x == 0) *p = 0;
}

__global__ __launch_bounds__(kScanThreads) void k_stats_one(TableView t, uint64_t arena_bytes,
                                                            uint64_t chunk, uint64_t ngroups,
                                                            ChunkSum *cs, WsHeader *hdr,
                                                            uint64_t fit_need) {
    stats_one_part<kScanThreads>(t, t.n, arena_bytes, chunk, ngroups, cs, hdr, fit_need,
                                 blockIdx.x);
}

// ---------------------------------------------------------------------------
// Tiles.  A run is a maximal sequence of moved live blocks; its destinations
// are contiguous (packed inside one segment).  Its tiles are the pieces of it
// inside each tile-size window: one starts at the run's first byte, and one at
// every multiple of T inside it.

// The last index k with a[k] <= x in a[0, m), or -1, for x = x0 (into
// out[0]) and x = x1 (into out[1]), a ascending: two searches side by
// side, 128 lanes each, every round testing 128 evenly spaced entries of
// the bracket at once (one memory round trip a round: three for a million
// entries, where one lane's bisection takes twenty).  Workgroup-uniform; 256
// lanes; barriers inside.
template <typename T>
__device__ inline void find_stretch(const T *a, int64_t m, uint64_t x0, uint64_t x1,
                                    int64_t *out) {
    __shared__ uint32_t s_cnt[4];
    __shared__ int64_t s_br[2][2];
    const uint32_t half = threadIdx.x >> 7, lane = threadIdx.x & 127, wave = threadIdx.x >> 6;
    const uint64_t x = half ? x1 : x0;
    if (lane == 0) {  // the bracket (lo, hi): a[lo] <= x < a[hi], a[-1] and a[m] beyond
        s_br[half][0] = -1;
        s_br[half][1] = m;
    }
    __syncthreads();
    for (;;) {
        const int64_t lo = s_br[half][0], hi = s_br[half][1];
        const int64_t lo_o = s_br[half ^ 1][0], hi_o = s_br[half ^ 1][1];
        if (hi - lo <= 1 && hi_o - lo_o <= 1) break;  // both done (uniform)
        const int64_t span = hi - lo - 1;  // candidates lo + 1 .. hi - 1
        const int64_t step = span > 0 ? (span + 127) / 128 : 1;
        const int64_t idx = lo + 1 + (int64_t)lane * step;
        const bool p = span > 0 && idx < hi && (uint64_t)a[idx] <= x;
        const uint64_t bal = __ballot(p);
        if ((threadIdx.x & 63) == 0) s_cnt[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        if (lane == 0 && span > 0) {  // the entries at or below x form a prefix
            const int64_t c = (int64_t)(s_cnt[2 * half] + s_cnt[2 * half + 1]);
            const int64_t nlo = c ? lo + 1 + (c - 1) * step : lo;
            const int64_t nhi = lo + 1 + c * step;
            s_br[half][0] = nlo;
            s_br[half][1] = nhi < hi ? nhi : hi;
        }
        __syncthreads();
    }
    if (lane == 0) out[half] = s_br[half][0];
}

// The remap's bucket index: ridx[b] = number of live blocks whose old offset
// is below b << w, for b in [0, nb]; one lane per entry, a binary search over
// the packed old offsets (workgroup blk covers entries [256 blk, ...)).  The
// workgroup's answers lie between those of its first and last bucket, found
// by find_stretch; when that stretch of old offsets is short (always, in a
// table of at most kIndexStage live blocks) it is staged in LDS with one
// memory round trip and searched there.
constexpr uint32_t kIndexStage = 2048;

// First k in [lo, hi) with a[k] >= x (hi if none).
__device__ inline uint64_t first_ge(const uint64_t *a, uint64_t lo, uint64_t hi, uint64_t x) {
    uint64_t len = hi - lo;
    while (len > 0) {
        const uint64_t half = len >> 1;
        if (a[lo + half] < x) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    return lo;
}

__device__ void remap_index_part(const uint64_t *__restrict__ live_src, uint64_t m, uint32_t w,
                                 uint64_t nb, uint32_t *ridx, uint64_t blk) {
    __shared__ uint64_t s_src[kIndexStage];
    __shared__ int64_t s_r[2];
    const uint64_t b0 = blk * kScanThreads;
    if (b0 > nb) return;  // (the whole workgroup)
    const uint64_t b1 = umin64(b0 + kScanThreads - 1, nb);  // >= 1: nb >= 1
    if (m <= kIndexStage) {
        if (threadIdx.x == 0) {
            s_r[0] = 0;
            s_r[1] = (int64_t)m;
        }
    } else {
        // blocks below x = (the last one at or below x - 1) + 1
        find_stretch(live_src, (int64_t)m, b0 ? (b0 << w) - 1 : 0, (b1 << w) - 1, s_r);
        __syncthreads();
        if (threadIdx.x == 0) {
            s_r[0] = b0 ? s_r[0] + 1 : 0;
            s_r[1] = s_r[1] + 1;
        }
    }
    __syncthreads();
    const uint64_t r0 = (uint64_t)s_r[0], r1 = (uint64_t)s_r[1];
    const bool staged = r1 - r0 <= kIndexStage;
    if (staged) {
        // every load issued before the first is stored: one round trip
        constexpr uint32_t kPer = kIndexStage / kScanThreads;
        uint64_t v[kPer] = {};
#pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            const uint64_t i = threadIdx.x + k * kScanThreads;
            if (i < r1 - r0) v[k] = live_src[r0 + i];
        }
#pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            const uint64_t i = threadIdx.x + k * kScanThreads;
            if (i < r1 - r0) s_src[i] = v[k];
        }
    }
    __syncthreads();
    const uint64_t b = b0 + threadIdx.x;
    if (b > b1) return;
    const uint64_t k = staged ? r0 + first_ge(s_src, 0, r1 - r0, b << w)
                              : first_ge(live_src, r0, r1, b << w);
    ridx[b] = (uint32_t)k;
}

struct BaseArgs {
    LiveView lv;
    const uint64_t *tpart, *twhole, *lbase;
    const StatPart *spart;
    uint64_t nb;
    TileChoice tiles;
    uint64_t max_tiles;
    uint32_t *tile_base;
    uint32_t *tgrp;     // first block of every 256th tile and of the last
    uint32_t *ridx;
    uint32_t rw;        // remap bucket width (log2 bytes)
    uint64_t rnb;       // remap buckets
    uint64_t arena_bytes;
    WsHeader *hdr;
    uint64_t *clear;  // set to zero (or null)
    uint64_t *arrive_post;  // the statistics header's count of finished workgroups
};

// Pass 3 of a plan.  Workgroups [0, nb): the tile size (every workgroup
// decides it the same way, from the same totals: the larger candidate when
// most moved bytes shift by less than kAutoSmallShift and enough bytes move,
// or when the smaller's tiles would not fit the workspace and the larger's
// do), then each of its live blocks' first tile index -- a block with no
// tile gets the index of the next tile that starts, so tile t belongs to the
// last block whose first index is <= t.  Workgroup nb takes the same
// decision and finishes the header beside them: statistics, tile count and
// size, the mover's fields.  The workgroups after it build the remap's
// bucket index.
// The tile size, decided the same way by every workgroup from the same
// totals: moved bytes, those shifting by less than kAutoSmallShift, and the
// tiles each candidate cuts (the larger always in a small arena or a table
// of small blocks, tc.always_b).  True: the larger candidate.
__device__ inline bool pick_larger(TileChoice tc, uint64_t moved, uint64_t small, uint64_t na,
                                   uint64_t nb, uint64_t max_tiles) {
    bool pick_b = tc.a != tc.b && (tc.always_b || (small * 2 > moved && moved >= kAutoMinMoved));
    if (tc.a != tc.b && (pick_b ? nb : na) > max_tiles && (pick_b ? na : nb) <= max_tiles)
        pick_b = !pick_b;
    return pick_b;
}

// The tile pass's stretches: block k, whose tiles are [run, run + c), is
// the first block of tile 256 q for each q with 256 q in that range
// (tgrp[q]) and, if it holds the last tile, of that one (tgrp[groups]).
// A lane writes a few such entries itself; a block with many (one of GiBs
// has hundreds) has them written by the whole wave, 64 at a time.  Every
// lane of the wave calls it (in: k is one of the workgroup's blocks).
__device__ inline void mark_groups(uint32_t *tgrp, bool in, uint64_t k, uint64_t run, uint64_t c,
                                   uint64_t n_tiles) {
    const uint64_t q0 = (run + 255) / 256;
    const uint64_t q1 = (in && c) ? (run + c + 255) / 256 : q0;  // groups q0 <= q < q1
    if (q1 - q0 <= 4) {
        for (uint64_t q = q0; q < q1; ++q) tgrp[q] = (uint32_t)k;
    }
    uint64_t many = __ballot(q1 - q0 > 4);
    const uint32_t lane = threadIdx.x & 63;
    while (many) {
        const int L = __ffsll((unsigned long long)many) - 1;
        const uint64_t b0 = __shfl(q0, L, 64), b1 = __shfl(q1, L, 64), bk = __shfl(k, L, 64);
        for (uint64_t q = b0 + lane; q < b1; q += 64) tgrp[q] = (uint32_t)bk;
        many &= many - 1;
    }
    if (in && c && run + c == n_tiles) tgrp[(n_tiles + 255) / 256] = (uint32_t)k;
}

__global__ __launch_bounds__(kScanThreads) void k_plan_bases(BaseArgs a) {
    __shared__ uint64_t sh[kScanThreads / 64];
    __shared__ uint64_t s_red[kStatSlots<kScanThreads>];
    __shared__ uint64_t s_before;
    WsHeader *hdr = a.hdr;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (a.clear) *a.clear = 0;
        *a.arrive_post = 0;  // for a one-launch statistics pass after this plan
    }
    const uint64_t g = blockIdx.x;
    if (g > a.nb) {
        const uint64_t m = hdr->live_blocks;
        if (plan_dead(hdr)) return;
        remap_index_part(a.lv.src, m, a.rw, a.rnb, a.ridx, g - a.nb - 1);
        return;
    }
    if (g == a.nb) {
        // workgroup nb finishes the header beside the others: every
        // per-workgroup statistic and tile count reduced at once (one
        // memory round trip, one reduction), the same tile decision, the
        // header written
        StatPart q{0, 0, 0, 0, kNone, kNone, kNone, 0};
        uint64_t x[4] = {0, 0, 0, 0};  // tiles and whole tiles, both candidates
        for (uint64_t j = threadIdx.x; j < a.nb; j += kScanThreads) {
            const StatPart p = a.spart[j];
            q.max_gap = umax64(q.max_gap, p.max_gap);
            q.gaps += p.gaps;
            q.moved_blocks += p.moved_blocks;
            q.moved_bytes += p.moved_bytes;
            q.min_moved_dst = umin64(q.min_moved_dst, p.min_moved_dst);
            q.min_size = umin64(q.min_size, p.min_size);
            q.min_fit = umin64(q.min_fit, p.min_fit);
            q.small_moved += p.small_moved;
            x[0] += a.tpart[j];
            x[1] += a.tpart[kMaxScanParts + j];
            x[2] += a.twhole[j];
            x[3] += a.twhole[kMaxScanParts + j];
        }
        const uint64_t max_end = hdr->max_live_end;
        if (plan_dead(hdr)) return;
        block_reduce_stats<kScanThreads>(q, x, s_red);
        const bool pick_b = pick_larger(a.tiles, q.moved_bytes, q.small_moved, x[0], x[1],
                                        a.max_tiles);
        if (threadIdx.x == 0) {
            stats_header(q, a.arena_bytes, max_end, kNone, hdr);
            hdr->n_tiles = pick_b ? x[1] : x[0];
            hdr->whole_tiles = pick_b ? x[3] : x[2];
            hdr->tile_bytes = pick_b ? a.tiles.b : a.tiles.a;
        }
        return;
    }
    uint64_t moved = 0, small = 0, pa, na, pb, nbt;
    uint64_t k_begin, k_end;
    if (a.nb <= 64) {
        // few workgroups before: the first wave takes one's counts a lane --
        // tiles for both candidates (their sums below g and totals), moved
        // and short-shift bytes -- and hands them out through LDS
        __shared__ uint64_t s_few[6];
        if (threadIdx.x < 64) {
            const uint32_t j = threadIdx.x;
            const bool in = j < a.nb;
            const uint64_t ta = in ? a.tpart[j] : 0, tb = in ? a.tpart[kMaxScanParts + j] : 0;
            const uint64_t mv = in ? a.spart[j].moved_bytes : 0;
            const uint64_t sm = in ? a.spart[j].small_moved : 0;
            const uint64_t ia = wave_incl_scan(ta, add_op), ib = wave_incl_scan(tb, add_op);
            const uint64_t ea = wave_shift_up(ia), eb = wave_shift_up(ib);
            const uint64_t m_all = wave_reduce(mv, add_op), s_all = wave_reduce(sm, add_op);
            if (j == g) {
                s_few[0] = ea;
                s_few[1] = eb;
            }
            if (j == 63) {  // lanes past nb add zero: the totals
                s_few[2] = ia;
                s_few[3] = ib;
                s_few[4] = m_all;
                s_few[5] = s_all;
            }
        }
        k_begin = a.lbase[g];
        k_end = a.lbase[g + 1];
        if (plan_dead(hdr)) return;
        __syncthreads();
        pa = wave_uniform(s_few[0]);
        pb = wave_uniform(s_few[1]);
        na = wave_uniform(s_few[2]);
        nbt = wave_uniform(s_few[3]);
        moved = wave_uniform(s_few[4]);
        small = wave_uniform(s_few[5]);
    } else {
        // every load that does not depend on another is issued before the
        // first is used (the header's outcome included): one memory round
        // trip where there were four
        const uint64_t j0 = (uint64_t)threadIdx.x * kPartsPer;
        uint64_t ta[kPartsPer], tb[kPartsPer];
#pragma unroll
        for (uint32_t k = 0; k < kPartsPer; ++k) {
            const bool in = j0 + k < a.nb;
            ta[k] = in ? a.tpart[j0 + k] : 0;
            tb[k] = in ? a.tpart[kMaxScanParts + j0 + k] : 0;
        }
        for (uint64_t j = threadIdx.x; j < a.nb; j += kScanThreads) {
            moved += a.spart[j].moved_bytes;
            small += a.spart[j].small_moved;
        }
        k_begin = a.lbase[g];
        k_end = a.lbase[g + 1];
        if (plan_dead(hdr)) return;
        {
            StatPart q{0, 0, 0, 0, kNone, kNone, kNone, 0};
            uint64_t x[4] = {moved, small, 0, 0};
            block_reduce_stats<kScanThreads>(q, x, s_red);
            moved = x[0];
            small = x[1];
        }
        sums_prefix(ta, g, sh, &s_before, pa, na);
        sums_prefix(tb, g, sh, &s_before, pb, nbt);
    }
    const bool pick_b = pick_larger(a.tiles, moved, small, na, nbt, a.max_tiles);
    const uint64_t T = pick_b ? a.tiles.b : a.tiles.a;
    const uint64_t n_tiles = pick_b ? nbt : na;
    if (n_tiles > a.max_tiles) return;  // the plan fails (the header says so)
    uint64_t carry = pick_b ? pb : pa;
    for (uint64_t s0 = k_begin; s0 < k_end; s0 += kScanTile) {
        const uint64_t k0 = s0 + (uint64_t)threadIdx.x * kScanItems;
        // the lane's blocks and the one before them (whether it moved says
        // whether a run starts), every load issued before the first is used
        uint64_t dd[kScanItems + 1], ss[kScanItems + 1], zz[kScanItems];
#pragma unroll
        for (uint32_t j = 0; j <= kScanItems; ++j) {
            const uint64_t k = k0 + j - 1;  // j = 0: the block before (none before block 0)
            dd[j] = 0;
            ss[j] = 0;
            if (k0 + j >= 1 && k < k_end) {
                dd[j] = a.lv.dst[k];
                ss[j] = a.lv.src[k];
            }
        }
#pragma unroll
        for (uint32_t j = 0; j < kScanItems; ++j) zz[j] = (k0 + j < k_end) ? a.lv.size[k0 + j] : 0;
        uint64_t c[kScanItems];
        uint64_t sum = 0;
#pragma unroll
        for (uint32_t j = 0; j < kScanItems; ++j) {
            // tiles starting inside block k0 + j (0 if it did not move)
            c[j] = 0;
            if (k0 + j < k_end && ss[j + 1] != dd[j + 1]) {
                const bool start = ss[j] == dd[j];  // the block before stayed (or is none)
                c[j] = tiles_of(dd[j + 1], zz[j], start, T);
            }
            sum += c[j];
        }
        uint64_t total;
        uint64_t run = carry + block_excl_sum<kScanThreads>(sum, total, sh);
        carry += total;
#pragma unroll
        for (uint32_t j = 0; j < kScanItems; ++j) {
            const bool in = k0 + j < k_end;
            if (in) a.tile_base[k0 + j] = (uint32_t)run;
            mark_groups(a.tgrp, in, k0 + j, run, c[j], n_tiles);
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

// The packed live arrays and the tile bases as the tile records read them:
// with STAGED, entries [lo, lo + cnt) from copies in LDS (the stretch of
// blocks a workgroup's tiles start in, and one on each side), any other from
// global memory; without, all from global memory.  The copies are addressed
// as LDS so that a read of either kind stays its own instruction.
typedef __attribute__((address_space(3))) const uint64_t lds_u64;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
template <bool STAGED>
struct LiveAt {
    LiveView lv;
    const uint32_t *tile_base;
    lds_u64 *s_dst, *s_src, *s_size;
    lds_u32 *s_tb;
    uint64_t lo, cnt;
    __device__ bool staged(uint64_t k) const { return STAGED && k - lo < cnt; }  // (k < lo wraps)
    __device__ uint64_t dst(uint64_t k) const { return staged(k) ? s_dst[k - lo] : lv.dst[k]; }
    __device__ uint64_t src(uint64_t k) const { return staged(k) ? s_src[k - lo] : lv.src[k]; }
    __device__ uint64_t size(uint64_t k) const { return staged(k) ? s_size[k - lo] : lv.size[k]; }
    __device__ uint64_t tb(uint64_t k) const { return staged(k) ? s_tb[k - lo] : tile_base[k]; }
    __device__ bool moved(uint64_t k) const { return src(k) != dst(k); }
};

// Every live block staged: all reads from LDS (entry k at k - lo), so the
// reads of a search step are issued together.
struct LiveLds {
    lds_u64 *s_dst, *s_src, *s_size;
    lds_u32 *s_tb;
    uint32_t lo;
    __device__ uint64_t dst(uint64_t k) const { return s_dst[(uint32_t)k - lo]; }
    __device__ uint64_t src(uint64_t k) const { return s_src[(uint32_t)k - lo]; }
    __device__ uint64_t size(uint64_t k) const { return s_size[(uint32_t)k - lo]; }
    __device__ uint64_t tb(uint64_t k) const { return s_tb[(uint32_t)k - lo]; }
    __device__ bool moved(uint64_t k) const { return src(k) != dst(k); }
};

// The same over a short array in LDS, in 32-bit arithmetic.
__device__ inline int32_t last_le32(const uint32_t *a, int32_t lo, int32_t hi, uint32_t x) {
    int32_t l = lo, h = hi;
    while (l < h) {
        const int32_t mid = l + ((h - l) >> 1);
        if (a[mid] <= x) l = mid + 1;
        else h = mid;
    }
    return l - 1;
}

// Where tile t starts, given its first block k (the last block whose first
// tile index tb_k is <= t).
template <typename LA>
__device__ inline uint64_t tile_start_at(const LA &lv, uint64_t k, uint64_t tb_k,
                                         uint64_t t, uint64_t T) {
    const uint64_t j = t - tb_k;
    const uint64_t a = lv.dst(k);
    const bool start = (k == 0) || !lv.moved(k - 1);
    const uint64_t lead = (start && (a & (T - 1))) ? 1 : 0;
    const uint64_t first_mult = (a + T - 1) & ~(T - 1);
    return (j < lead) ? a : first_mult + (j - lead) * T;
}

// The tile holding destination byte q of moved block b (tiles cut each run
// at its start and at every multiple of T).
template <typename LA>
__device__ inline uint64_t tile_of(const LA &lv, uint64_t b, uint64_t q, uint64_t T) {
    const uint64_t a = lv.dst(b);
    const uint64_t A = (a + T - 1) & ~(T - 1);
    const bool start = (b == 0) || !lv.moved(b - 1);
    const uint64_t lead = (start && (a & (T - 1))) ? 1 : 0;
    const uint64_t tb = lv.tb(b);
    if (q >= A) return tb + lead + div_tile(q - A, T);
    // q lies in the window block b starts in: block b's own first tile if it
    // starts a run there, else the tile that began earlier in the run
    return lead ? tb : tb - 1;
}

// Tile t's record, given its start t0, its first block and its end bound
// (the next tile's start or the window's end).  [t0, t1) = the run's bytes
// from t0 up to the bound or the run's end.  A tile may write only once
// every tile whose sources overlap [t0, t1) has read them.  Sources rise
// strictly with destinations (src = dst + shift, shifts never negative,
// order kept), so the destinations whose sources lie in [t0, t1) are at most
// t1 - t0 consecutive live bytes, all at or below [t0, t1): their tiles are
// a short range ending at or before this one.  ridx: the remap's bucket
// index (bucket width 2^w), which narrows the search for the first such
// block, or null to search all m blocks.
template <typename LA>
__device__ inline TileRec tile_record(const LA &lv, uint64_t m, uint64_t t, uint64_t t0,
                                      uint64_t first, uint64_t bound, uint64_t T,
                                      const uint32_t *ridx, uint32_t w) {
    // Two searches that do not depend on each other run in one loop, the
    // loads of a step issued together (each step is a memory round trip
    // unless the blocks are staged):
    //  * the last block of the run inside [t0, bound): the blocks after
    //    first that start below bound and moved form a prefix -- gallop
    //    (doubling), then bisect; the end of the last one found so far is
    //    kept, so t1 needs no further load;
    //  * the first block whose source ends above t0 (the first whose source
    //    can overlap [t0, t1)).  The remap index narrows it to the blocks
    //    starting in t0's bucket and the one before them: an earlier block
    //    ends before the bucket starts, and the first block of the next
    //    bucket already ends above t0.
    int64_t lo = 0, hi = (int64_t)m;
    if (ridx) {
        const uint64_t bk = t0 >> w;
        const uint32_t r0 = ridx[bk], r1 = ridx[bk + 1];
        lo = r0 ? (int64_t)r0 - 1 : 0;
        hi = (int64_t)r1;
    }
    uint64_t last = first, stride = 1;
    uint64_t last_end = lv.dst(first) + lv.size(first);
    bool doubling = true;
    for (;;) {
        const bool g_on = stride > 0;
        const bool s_on = lo < hi;
        if (!g_on && !s_on) break;
        const uint64_t gi = last + stride;
        const int64_t mid = lo + ((hi - lo) >> 1);
        bool g_ok = false;
        uint64_t g_end = 0;
        if (g_on && gi < m) {
            const uint64_t d = lv.dst(gi), sz = lv.size(gi), sr = lv.src(gi);
            g_ok = (d < bound) & (sr != d);  // starts below bound, moved
            g_end = d + sz;
        }
        bool s_right = false;
        if (s_on) s_right = lv.src(mid) + lv.size(mid) <= t0;
        if (g_on) {
            if (g_ok) {
                last = gi;
                last_end = g_end;
            }
            if (doubling && g_ok) {
                stride <<= 1;
            } else {
                doubling = false;
                stride >>= 1;
            }
        }
        if (s_on) {
            if (s_right) lo = mid + 1;
            else hi = mid;
        }
    }
    const uint64_t t1 = umin64(bound, last_end);
    uint32_t dep_lo = 1, dep_hi = 0;  // empty
    if (lo < (int64_t)m && t > 0) {
        const uint64_t j = (uint64_t)lo;
        const uint64_t sj = lv.src(j);
        if (sj < t1) {
            const uint64_t q_lo = lv.dst(j) + (t0 > sj ? t0 - sj : 0);
            const uint64_t u_lo = tile_of(lv, j, q_lo, T);
            // ... and the last block whose source starts below t1 (gallop from j)
            uint64_t c = j;
            stride = 1;
            while (c + stride < m && lv.src(c + stride) < t1) {
                c += stride;
                stride <<= 1;
            }
            for (; stride > 0; stride >>= 1)
                if (c + stride < m && lv.src(c + stride) < t1) c += stride;
            const uint64_t sc = lv.src(c);
            const uint64_t q_hi = lv.dst(c) + umin64(lv.size(c), t1 - sc) - 1;
            uint64_t u_hi = tile_of(lv, c, q_hi, T);
            if (u_hi > t - 1) u_hi = t - 1;
            if (u_lo <= u_hi) {
                dep_lo = (uint32_t)u_lo;
                dep_hi = (uint32_t)u_hi;
            }
        }
    }
    return TileRec{t0, t1, lv.src(first) - lv.dst(first), (uint32_t)first, (uint32_t)last,
                   dep_lo, dep_hi, 0};
}

// Pass 4: one lane per tile, each writing its record (tile_record).
//
// Each tile's first block is the last block whose first tile index is <= t
// (a search over tile_base).  The workgroup's tiles [tb, tb + 256) -- and the
// tile after them, whose start bounds the last one -- have their first blocks
// in one stretch of tile_base.  When it is short, that stretch of tile_base
// and of the packed live arrays (with one block on each side) is staged in
// LDS with one memory round trip, and the searches for each tile's first
// block, its start and its run read there; a small plan stages every live
// block and reads global memory only to stage.  Each lane also leaves its
// tile's start in LDS for the lane before it.
constexpr uint32_t kTileStage = 2048;  // blocks of the stretch staged per workgroup
// Plans of at most this many tiles stage the live arrays: 512 workgroups,
// two on each compute unit of a 256-CU device.
constexpr uint64_t kStageTileLimit = 512ull * 256;

// STAGE: the live arrays are staged too (58 KiB of LDS, two workgroups per
// compute unit); without, tile_base alone (8 KiB).  Staging pays when the
// plan's tiles take few workgroups, which then all run at once.
template <bool STAGE>
__global__ __launch_bounds__(256) void k_tiles(LiveView lv, const uint32_t *tile_base,
                                               const uint32_t *tgrp, const WsHeader *hdr,
                                               uint64_t max_tiles, const uint32_t *ridx,
                                               uint32_t w, TileRec *tiles, uint32_t *flags) {
    constexpr uint32_t kCap = kTileStage + 2;
    constexpr uint32_t kLiveCap = STAGE ? kCap : 1;
    __shared__ uint32_t s_tb[kCap];
    __shared__ uint64_t s_dst[kLiveCap], s_src[kLiveCap], s_size[kLiveCap];
    __shared__ uint64_t s_t0[257];
    // the first blocks of the workgroup's first tile and of the last tile
    // whose start it needs (the bases pass recorded them; loaded beside the
    // header: the array holds an entry past the grid's last workgroup)
    const uint32_t g_lo = tgrp[blockIdx.x], g_hi = tgrp[blockIdx.x + 1];
    const uint64_t n_tiles = hdr->n_tiles, m = hdr->live_blocks, T = hdr->tile_bytes;
    if (plan_dead(hdr) | (n_tiles > max_tiles)) return;  // plan fails
    const uint64_t tb = (uint64_t)blockIdx.x * 256;
    if (tb >= n_tiles) return;  // (the whole workgroup)
    const uint64_t t = tb + threadIdx.x;
    const uint64_t te = umin64(tb + 256, n_tiles);
    // the stretch of tile_base holding the first blocks of tiles [tb, tq],
    // tq = te or the last tile: a small plan takes all of its blocks (and
    // then reads them through the LDS-only accessor)
    const bool whole = m <= kTileStage;
    const int64_t k_lo = whole ? 0 : (int64_t)g_lo;
    const int64_t k_hi = whole ? (int64_t)m - 1 : (int64_t)g_hi;
    const bool staged = k_hi - k_lo < (int64_t)kTileStage;
    // staged: blocks [s_lo, s_lo + s_cnt) -- the stretch, the block before it
    // (a tile's start reads the block before its first) and the one after
    // it (a run's last block may follow the stretch)
    const uint64_t s_lo = (staged && k_lo > 0) ? (uint64_t)k_lo - 1 : 0;
    const uint64_t s_cnt = staged ? umin64((uint64_t)k_hi + 2, m) - s_lo : 0;
    if (staged) {
        // every load issued before the first is stored: one round trip
        constexpr uint32_t kPer = (kCap + 255) / 256;
        uint64_t vd[kPer] = {}, vs[kPer] = {}, vz[kPer] = {};
        uint32_t vt[kPer] = {};
#pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            const uint64_t i = threadIdx.x + k * 256;
            if (i < s_cnt) {
                vt[k] = tile_base[s_lo + i];
                if constexpr (STAGE) {
                    vd[k] = lv.dst[s_lo + i];
                    vs[k] = lv.src[s_lo + i];
                    vz[k] = lv.size[s_lo + i];
                }
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            const uint64_t i = threadIdx.x + k * 256;
            if (i < s_cnt) {
                s_tb[i] = vt[k];
                if constexpr (STAGE) {
                    s_dst[i] = vd[k];
                    s_src[i] = vs[k];
                    s_size[i] = vz[k];
                }
            }
        }
    }
    __syncthreads();
    const LiveAt<STAGE> la{lv, tile_base, (lds_u64 *)s_dst, (lds_u64 *)s_src, (lds_u64 *)s_size,
                           (lds_u32 *)s_tb, s_lo, s_cnt};
    const LiveLds ll{(lds_u64 *)s_dst, (lds_u64 *)s_src, (lds_u64 *)s_size, (lds_u32 *)s_tb,
                     (uint32_t)s_lo};
    const bool all = STAGE && s_lo == 0 && s_cnt == m;  // every live block staged
    // first block of tile u among blocks [k0, k_hi] (k_lo <= k0), and its
    // first tile index
    const auto first_of = [&](uint64_t u, int64_t k0, uint64_t *tb_k) -> uint64_t {
        if (staged) {
            const int32_t r = last_le32(s_tb, (int32_t)(k0 - (int64_t)s_lo),
                                        (int32_t)(k_hi - (int64_t)s_lo + 1), (uint32_t)u);
            *tb_k = s_tb[r];
            return s_lo + (uint64_t)r;
        }
        const int64_t k = last_le(tile_base, k0, k_hi + 1, u);
        *tb_k = tile_base[k];
        return (uint64_t)k;
    };
    const auto start_of = [&](uint64_t k, uint64_t tb_k, uint64_t u) -> uint64_t {
        return all ? tile_start_at(ll, k, tb_k, u, T) : tile_start_at(la, k, tb_k, u, T);
    };
    uint64_t first = 0, t0 = 0, tb_k;
    if (t < te) {
        first = first_of(t, k_lo, &tb_k);
        t0 = start_of(first, tb_k, t);
        s_t0[threadIdx.x] = t0;
    }
    if (threadIdx.x == 255 && te < n_tiles) {  // the tile after the workgroup's: its
        // first block is at or after this lane's
        const uint64_t k = first_of(te, (int64_t)first, &tb_k);
        s_t0[256] = start_of(k, tb_k, te);
    }
    __syncthreads();
    if (t >= n_tiles) return;
    uint64_t bound = (t0 & ~(T - 1)) + T;
    if (t + 1 < n_tiles) bound = umin64(bound, s_t0[threadIdx.x + 1]);
    tiles[t] = all ? tile_record(ll, m, t, t0, first, bound, T, ridx, w)
                   : tile_record(la, m, t, t0, first, bound, T, ridx, w);
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

struct SelCand {
    uint64_t c, k, l;
};
__device__ inline SelCand sel_op(const SelCand &a, const SelCand &b) {
    return sel_better(b.c, b.k, a.c, a.k) ? b : a;
}

// Workgroup arg-min of (cost, k) carrying l, through LDS (NT threads).
template <int NT>
__device__ inline void sel_reduce(uint64_t &c, uint64_t &k, uint64_t &l, uint64_t *sh) {
    constexpr int NW = NT / 64;
    const SelCand best = wave_reduce(SelCand{c, k, l}, sel_op);
    c = best.c;
    k = best.k;
    l = best.l;
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
                uint64_t epoch, uint64_t fit_need, uint64_t *clear, hipStream_t s) {
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    ScanPart *part = reinterpret_cast<ScanPart *>(ws + L.part);
    StatPart *spart = reinterpret_cast<StatPart *>(ws + L.spart);
    DownArgs d{};
    d.t = t;
    d.win = win;
    d.part = part;
    d.nb = L.n_scan_blocks;
    d.ngroups = d.nb ? d.nb : 1;
    d.chunk = L.scan_chunk;
    d.hdr = hdr;
    d.new_offset = new_offset;
    d.lo = LiveOut{reinterpret_cast<uint64_t *>(ws + L.live_dst),
                   reinterpret_cast<uint64_t *>(ws + L.live_src),
                   reinterpret_cast<uint64_t *>(ws + L.live_size),
                   reinterpret_cast<uint8_t *>(ws + L.live_pin),
                   reinterpret_cast<uint64_t *>(ws + L.live_z),
                   reinterpret_cast<uint32_t *>(ws + L.live_pc),
                   nullptr, nullptr, nullptr, nullptr, 0};
    if (remap_ent(arena_bytes, t.n)) {
        d.lo.ent = reinterpret_cast<RemapEnt *>(ws + L.live_rec);
        d.lo.key_mask = (1ull << remap_shift(arena_bytes, t.n)) - 1;
    } else if (remap_rec32(arena_bytes)) {
        d.lo.rec32 = reinterpret_cast<LiveRec32 *>(ws + L.live_rec);
    } else {
        d.lo.rec = reinterpret_cast<LiveRec *>(ws + L.live_rec);
    }
    if (!d.lo.ent && remap_keys32(arena_bytes, t.n)) {
        d.lo.key = reinterpret_cast<uint32_t *>(ws + L.live_key);
        d.lo.key_mask = (1ull << remap_shift(arena_bytes, t.n)) - 1;
    }
    d.spart = spart;
    d.tpart = reinterpret_cast<uint64_t *>(ws + L.tpart);
    d.twhole = reinterpret_cast<uint64_t *>(ws + L.twhole);
    d.lbase = reinterpret_cast<uint64_t *>(ws + L.lbase);
    d.tiles = tiles;
    d.fit_need = fit_need;
    d.epoch = epoch;
    d.arena_bytes = arena_bytes;

    // pass 1: aggregates
    if (d.nb) {
        hipLaunchKernelGGL(k_scan_partials, dim3((uint32_t)d.nb), dim3(kScanThreads), 0, s, t,
                           arena_bytes, win, (uint64_t)L.scan_chunk, part);
        AC_TRY(hipGetLastError());
    }
    // pass 2: each workgroup's prefix, then its entries
    if (outputs == kOutNew)
        hipLaunchKernelGGL(k_scan_down<kOutNew>, dim3((uint32_t)d.ngroups), dim3(kScanThreads), 0,
                           s, d);
    else
        hipLaunchKernelGGL(k_scan_down<kOutSelect>, dim3((uint32_t)d.ngroups), dim3(kScanThreads),
                           0, s, d);
    AC_TRY(hipGetLastError());
    if (!(outputs & kOutNew)) return hipSuccess;  // a selection scan ends there
    // pass 3: tile size, the blocks' first tiles and the header's finish;
    // the remap index beside them
    const LiveView lv = live_view(ws, L);
    uint32_t *ridx = reinterpret_cast<uint32_t *>(ws + L.ridx);
    uint32_t *tile_base = reinterpret_cast<uint32_t *>(ws + L.tile_base);
    BaseArgs b{};
    b.lv = lv;
    b.tpart = d.tpart;
    b.twhole = d.twhole;
    b.lbase = d.lbase;
    b.spart = spart;
    b.nb = d.ngroups;
    b.tiles = tiles;
    b.max_tiles = L.max_tiles;
    b.tile_base = tile_base;
    b.tgrp = reinterpret_cast<uint32_t *>(ws + L.tgrp);
    b.ridx = ridx;
    b.rw = remap_shift(arena_bytes, t.n);
    b.rnb = remap_buckets(arena_bytes, t.n);
    b.arena_bytes = arena_bytes;
    b.hdr = hdr;
    b.clear = clear;
    b.arrive_post = &reinterpret_cast<WsHeader *>(ws + L.post)->arrive;
    const uint64_t rblocks = (b.rnb + 1 + kScanThreads - 1) / kScanThreads;
    hipLaunchKernelGGL(k_plan_bases, dim3((uint32_t)(d.ngroups + 1 + rblocks)), dim3(kScanThreads), 0,
                       s, b);
    AC_TRY(hipGetLastError());
    // pass 4: the tile records, a grid for the whole capacity (each lane
    // checks the device-side tile count: no host round trip)
    TileRec *trec = reinterpret_cast<TileRec *>(ws + L.tiles);
    uint32_t *flags = reinterpret_cast<uint32_t *>(ws + L.flags);
    const uint64_t grid = (L.max_tiles + 255) / 256;
    if (grid) {
        // at most arena / T tiles cut at multiples of T, and one more per run
        const uint32_t t_min = tiles.a < tiles.b ? tiles.a : tiles.b;
        const uint64_t bound = arena_bytes / t_min + t.n;
        if (bound <= kStageTileLimit)
            hipLaunchKernelGGL(k_tiles<true>, dim3((uint32_t)grid), dim3(256), 0, s, lv, tile_base,
                               b.tgrp, hdr, L.max_tiles, ridx, b.rw, trec, flags);
        else
            hipLaunchKernelGGL(k_tiles<false>, dim3((uint32_t)grid), dim3(256), 0, s, lv,
                               tile_base, b.tgrp, hdr, L.max_tiles, ridx, b.rw, trec, flags);
        AC_TRY(hipGetLastError());
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_scan(const TableView &t, uint64_t arena_bytes, uint8_t *ws, const WsLayout &L,
                       uint64_t *new_offset, int outputs, TileChoice tiles, uint64_t epoch,
                       uint64_t fit_need, uint64_t *clear, hipStream_t s) {
    return queue_scan(t, arena_bytes, ws, L, new_offset, outputs, nullptr, tiles, epoch,
                      fit_need, clear, s);
}

hipError_t launch_targeted(const TableView &t, uint64_t arena_bytes, uint64_t request,
                           uint8_t *ws, const WsLayout &L, uint64_t *new_offset,
                           TileChoice tiles, uint64_t epoch, uint64_t *clear, hipStream_t s) {
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    const uint64_t *src = reinterpret_cast<const uint64_t *>(ws + L.live_src);
    const uint64_t *size = reinterpret_cast<const uint64_t *>(ws + L.live_size);
    const uint64_t *z = reinterpret_cast<const uint64_t *>(ws + L.live_z);
    const uint32_t *pc = reinterpret_cast<const uint32_t *>(ws + L.live_pc);
    SelPart *sp = reinterpret_cast<SelPart *>(ws + L.selpart);
    AC_TRY(queue_scan(t, arena_bytes, ws, L, nullptr, kOutSelect, nullptr, tiles, epoch,
                      kNone, nullptr, s));
    // candidates: every last hole l in [0, m], m <= n
    hipLaunchKernelGGL(k_select, dim3((uint32_t)L.n_sel_blocks), dim3(kSelThreads), 0, s, src, z,
                       pc, hdr, arena_bytes, request, sp);
    AC_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_select_finish, dim3(1), dim3(kSpineThreads), 0, s, sp, L.n_sel_blocks,
                       src, size, z, arena_bytes, hdr);
    AC_TRY(hipGetLastError());
    return queue_scan(t, arena_bytes, ws, L, new_offset, kOutNew, &hdr->win_begin, tiles,
                      epoch, kNone, clear, s);
}

hipError_t launch_stats_one(const TableView &t, uint64_t arena_bytes, uint8_t *ws,
                            const WsLayout &L, uint64_t fit_need, bool after_plan,
                            hipStream_t s) {
    const uint64_t ngroups = L.n_scan_blocks ? L.n_scan_blocks : 1;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    if (!after_plan && ngroups > 1) {
        hipLaunchKernelGGL(k_clear_u64, dim3(1), dim3(64), 0, s, &hdr->arrive);
        AC_TRY(hipGetLastError());
    }
    hipLaunchKernelGGL(k_stats_one, dim3((uint32_t)ngroups), dim3(kScanThreads), 0, s, t,
                       arena_bytes, (uint64_t)L.scan_chunk, ngroups,
                       reinterpret_cast<ChunkSum *>(ws + L.csum), hdr, fit_need);
    return hipGetLastError();
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

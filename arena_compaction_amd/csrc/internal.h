// internal.h -- workspace layout and kernel launchers shared by the library's
// own sources (api.cpp, plan.hip, move.hip, remap.hip).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

// Nothing declared here is part of the library's interface.
#pragma GCC visibility push(hidden)

namespace ac {

constexpr uint32_t kScanThreads = 256;          // threads per scan workgroup
constexpr uint32_t kScanItems = 4;              // table entries per thread (measured: 4 beats 2 and 8)
constexpr uint32_t kScanTile = kScanThreads * kScanItems;  // entries per workgroup step
// The scans run on a fixed grid: at most this many workgroups, each taking a
// contiguous chunk of whole steps.  Their per-workgroup results then fit in
// regions of fixed size at the front of the workspace, which is all a
// statistics pass writes besides its header: it can measure a table of any
// size while the workspace holds a plan, whose arrays all lie behind them.
constexpr uint32_t kMaxScanParts = 1024;
constexpr uint32_t kSpineThreads = 256;         // single-workgroup passes (no spills)
// Mover workgroup: 512 lanes, a 64 KiB tile being 8 vectors of 16 B per
// lane (measured on the 80 GiB workload, one workgroup per CU: 512 lanes
// 86.3-86.6%, 256 lanes 85.9-86.2%, 1,024 lanes 86.0%).
constexpr uint32_t kMoveThreads = 512;
// Tables of small blocks (under 8 KiB of arena per entry, so a tile holds
// several blocks between free ones) take 1,024 lanes: on the 4 GiB heap of
// 32-4,096 B blocks 78.5% against 75.7-76.0% at 512, while the large-block
// workloads lose 0.3-0.4 points with them.
constexpr uint32_t kMoveThreadsSmallBlocks = 1024;
constexpr uint64_t kSmallBlockBytes = 8192;
inline bool move_small_blocks(uint64_t arena_bytes, uint64_t n) {
    return n && arena_bytes / n < kSmallBlockBytes;
}
constexpr uint32_t kDefaultTile = 65536;
// With no tile size given, the plan picks one on the device from the shifts
// it finds: 64 KiB tiles, or 128 KiB when most moved bytes shift by less
// than kAutoSmallShift and at least kAutoMinMoved bytes move.  A tile whose
// sources the tile it depends on has not yet read waits about a fixed time,
// and with shifts that short (within the window of tiles in flight at once,
// ~16 MiB of 64 KiB tiles on 256 compute units) most do.  128 KiB tiles are
// moved two per workgroup in flight, so a tile looks at its dependencies
// only after the next tile's loads have gone out, and by then they have
// nearly always published.  Measured (mover only, share of the 8 TB/s
// peak): eight 1 GiB blocks each above a 4 KiB-1 MiB hole, 62% with 64 KiB
// tiles, 77% with 256 KiB tiles one at a time, 83% with 128 KiB two at a
// time; sixty-four 1 GiB blocks above 4 KiB-64 MiB holes (most bytes
// shifting far), 85% with 64 KiB tiles and 83% with 128 KiB two at a time.
constexpr uint32_t kAutoTileSmall = 65536;
constexpr uint32_t kAutoTileLarge = 131072;
constexpr uint64_t kAutoSmallShift = 8ull << 20;
constexpr uint64_t kAutoMinMoved = 64ull << 20;
// The plan picks 128 KiB whatever the shifts in two cases.  An arena of at
// most kAutoMinMoved bytes: a step that small is bound by latency, and half
// as many tiles, two per workgroup in flight, wait less (the 64 MiB table
// of 4,096 blocks: one call 67.9-68.9 -> 64.8-65.8 us, 381 tiles of which
// 153-159 late -> 191 of which 36-46).  A table of small blocks (the
// 1,024-lane mover, one tile at a time): each tile's record and block table
// are fetched once for twice the bytes (the 4 GiB table of 32 B-4 KiB
// blocks: mover 77.9 -> 78.6% of peak, one call 1.001-1.006 -> 0.974-0.979
// ms).  The one-call path then launches that mover alone.
inline bool auto_larger_always(uint64_t arena_bytes, uint64_t n) {
    return arena_bytes <= kAutoMinMoved || move_small_blocks(arena_bytes, n);
}

// The tile sizes a plan counts tiles for: a == b for a size the caller gave.
struct TileChoice {
    uint32_t a, b;
    uint32_t always_b;  // a != b: b whatever the shifts (auto_larger_always)
};
// Mover workgroups per compute unit when the caller gives no tuning: one,
// which keeps one narrow window of tiles in flight (two 512-lane workgroups
// per CU: 80.5% on the 80 GiB workload).
constexpr uint32_t kDefaultWgPerCu = 1;
constexpr uint32_t kDefaultNontemporal = 1; // streaming loads and stores
constexpr uint32_t kMinTile = 256;
constexpr uint32_t kMaxTile = 262144;
constexpr uint32_t kDefaultSpinLog2 = 22;
constexpr uint64_t kNone = ~0ull;
// Tile indices and the mover's ticket are 32-bit.  Every mover workgroup
// makes one last claim past the end, so tiles plus the grid must stay below
// 2^32: tiles are capped here and the grid at kMaxMoveGrid.
constexpr uint64_t kMaxTiles = 0xFFFF0000ull;
constexpr uint64_t kMaxMoveGrid = 0xFFFFull;

// Device-resident plan header (first 256 bytes of the workspace).
struct alignas(256) WsHeader {
    uint64_t live_bytes;     // LT: sum of live sizes (pinned included)
    uint64_t live_blocks;    // m (pinned included)
    uint64_t max_live_end;   // end of the highest live block (0 if none)
    uint64_t bad_key;        // (index << 3) | reason of the first bad entry, kNone if valid
    uint64_t largest_hole;   // longest run outside live blocks, tail included
    uint64_t hole_count;     // number of such runs
    uint64_t moved_blocks;
    uint64_t moved_bytes;
    uint64_t pinned_blocks;
    uint64_t min_live_size;  // kNone if no live block
    uint64_t move_begin;     // lowest destination written by the move (kNone if none)
    uint64_t n_tiles;        // mover tiles
    uint64_t epoch;          // plan epoch, checked by the mover
    uint32_t ticket;         // mover tile ticket counter
    uint32_t status;         // mover status bits (kStatus*)
    // targeted plans: the window chosen for the request (kWin*)
    uint64_t win_state;
    uint64_t win_begin;      // [win_begin, win_end): the window's bytes
    uint64_t win_end;
    uint64_t win_hole;       // free bytes inside it (the hole it frees)
    uint64_t win_moved;      // live bytes inside it (the bytes that move)
    uint64_t fit_offset;     // first fit: lowest hole start holding the request
    uint64_t whole_tiles;    // tiles that are one whole window of one block
    // The mover's wait counters (zeroed by the plan): tiles whose dependency
    // flags were not all seen set behind their loads, tiles that then read
    // a flag unset at least once, and all such unset reads.
    uint64_t late_tiles;
    uint64_t waited_tiles;
    uint64_t polls;
    uint64_t tile_bytes;     // the plan's tile size (chosen on the device when auto)
    uint64_t small_moved;    // moved bytes whose shift is below kAutoSmallShift
    // statistics passes: workgroups done (cleared by the aggregates pass,
    // or for the one-launch pass by the plan before it, and by the last
    // workgroup once it has completed the header)
    uint64_t arrive;
    uint64_t pad[5];
};
static_assert(sizeof(WsHeader) == 256, "header size");

constexpr uint32_t kStatusTimeout = 1u;   // a wait gave up (the watchdog)
constexpr uint32_t kStatusCapacity = 2u;  // a tile met more blocks than its LDS holds
constexpr uint32_t kStatusCorrupt = 4u;   // a tile's record or blocks lie outside the
                                          // arena or the plan's arrays: nothing moved
// Wait-path testing knob: at most this many sleeps per stalled tile.
constexpr uint32_t kMaxStallSleeps = 4096;

constexpr uint64_t kWinNone = 0;   // not a targeted plan
constexpr uint64_t kWinFound = 1;
constexpr uint64_t kWinNoFit = 2;  // no window frees the request: plan nothing

// Scan outputs (bit flags).
constexpr int kOutNew = 1;     // new offsets, packed live arrays, plan epoch
constexpr int kOutSelect = 2;  // packed old offset and size, live-byte and
                               // pinned-count prefixes; plan epoch (bumped so
                               // an older plan in the workspace goes stale)

// Element of the plan's scan over table entries.  v is a segmented sum: a
// pinned entry resets it to its own end (the start of the next segment), a
// movable live entry adds its size.  The other fields are plain sum / max.
struct Agg {
    uint64_t v;      // packed position inside the current segment
    uint64_t mx;     // highest live end
    uint64_t cnt;    // live entries
    uint64_t lsum;   // live bytes
    uint64_t pcnt;   // pinned entries
    uint32_t r;      // a pinned entry (segment reset) is inside
    uint32_t pad;
};

// Per scan-workgroup aggregate plus the smallest bad-entry key seen.
struct ScanPart {
    Agg a;
    uint64_t bad_key;
};

// Per selection-workgroup best window: fewest moved bytes, then lowest
// first hole; k and l are the first and last hole (hole q lies just below
// live block q, hole m is the tail).
struct SelPart {
    uint64_t cost;
    uint64_t k;
    uint64_t l;
    uint64_t pad;
};
constexpr uint32_t kSelThreads = 256;  // one candidate last hole per thread

// Per scan-workgroup hole / move statistics.
struct StatPart {
    uint64_t max_gap;
    uint64_t gaps;
    uint64_t moved_blocks;
    uint64_t moved_bytes;
    uint64_t min_moved_dst;
    uint64_t min_size;
    uint64_t min_fit;   // lowest start of a hole below a live block holding fit_need
    uint64_t small_moved;  // moved bytes whose shift is below kAutoSmallShift
};

// One mover tile: the destination bytes [t0, t1) -- a piece of one run of
// moved blocks, inside one tile-size window -- the live blocks first..last it
// covers, the shift of its first block, and the earlier tiles whose sources
// overlap [t0, t1) (dep_lo > dep_hi means none).
struct alignas(16) TileRec {
    uint64_t t0;
    uint64_t t1;
    uint64_t shift0;
    uint32_t first_block;
    uint32_t last_block;
    uint32_t dep_lo;
    uint32_t dep_hi;
    uint64_t pad;
};
static_assert(sizeof(TileRec) == 48, "tile record size");

// One live block as the handle remap reads it, once its search has found
// the last block starting at or below a handle h: h lies in it iff h < end,
// and then maps to h - shift.  16 bytes; arenas below 2^37 bytes use the
// 8-byte LiveRec32 below, or the 16-byte key-and-record RemapEnt.
struct alignas(16) LiveRec {
    uint64_t end;    // old offset + size
    uint64_t shift;  // old offset - new offset (0 for a block that stays)
};
static_assert(sizeof(LiveRec) == 16, "live record size");

// The same record in 32-byte units, 8 bytes, for arenas below 2^37 bytes
// (every offset and size is a multiple of 32, so nothing is lost and the
// old end fits in 32 bits): half the cache footprint of LiveRec.  Used when
// the remap's buckets are wider than 2^32 bytes (a few blocks in an arena of
// 2^35 bytes or more); narrower buckets put it beside the key in RemapEnt.
struct alignas(8) LiveRec32 {
    uint32_t end32;    // (old offset + size) / 32
    uint32_t shift32;  // (old offset - new offset) / 32
};
static_assert(sizeof(LiveRec32) == 8, "packed live record size");
inline bool remap_rec32(uint64_t arena_bytes) { return arena_bytes < (1ull << 37); }

// Remap index: the arena is cut into buckets of 2^w bytes, at most
// remap_bucket_cap(n) of them, and ridx[b] counts the live blocks starting
// below bucket b (entries 0 .. buckets).  At most 2^20 buckets (4 MiB of
// index): on the 4 GiB heap of a million live blocks the remap took 254 us
// with 2^18, 208 us with 2^20 and 242 us with 2^22 (whose index no longer
// stays in cache and takes twice as long to build).
inline uint64_t remap_bucket_cap(uint64_t n) {
    uint64_t c = 16;
    while (c < 2 * n + 2 && c < (1ull << 20)) c <<= 1;
    return c;
}
inline uint32_t remap_shift(uint64_t arena_bytes, uint64_t n) {
    const uint64_t cap = remap_bucket_cap(n);
    uint32_t w = 5;
    while ((arena_bytes >> w) >= cap) ++w;
    return w;
}
inline uint64_t remap_buckets(uint64_t arena_bytes, uint64_t n) {
    return (arena_bytes >> remap_shift(arena_bytes, n)) + 1;
}
// With buckets of at most 2^32 bytes the search inside a bucket compares
// 32-bit keys, each live block's old offset inside its bucket, instead of
// the 64-bit offsets: half the bytes per probe.  Wider buckets (a tiny
// table in an arena above 2^35 bytes) search the 64-bit offsets.
inline bool remap_keys32(uint64_t arena_bytes, uint64_t n) {
    return remap_shift(arena_bytes, n) <= 32;
}

// Both 32-bit forms at once (arenas below 2^37 bytes, buckets of at most
// 2^32): a live block's search key and its record side by side in 16 bytes,
// so the probe that finds the block has read its record too.
struct alignas(16) RemapEnt {
    uint32_t key;      // old offset inside its bucket
    uint32_t end32;    // (old offset + size) / 32
    uint32_t shift32;  // (old offset - new offset) / 32
    uint32_t pad;
};
static_assert(sizeof(RemapEnt) == 16 && sizeof(RemapEnt) <= sizeof(LiveRec),
              "remap entries share the record region");
inline bool remap_ent(uint64_t arena_bytes, uint64_t n) {
    return remap_rec32(arena_bytes) && remap_keys32(arena_bytes, n);
}

constexpr size_t kPerTileBytes = sizeof(TileRec) + sizeof(uint32_t);

struct WsLayout {
    // fixed part (depends on n only)
    size_t header, post, part, spart, csum, tpart, twhole, lbase, live_dst, live_src, live_size,
        live_pin, tile_base, live_z, live_pc, selpart, live_rec, live_key, ridx, fixed;
    // tile part (depends on the tile capacity)
    // tgrp: the first block of every 256th tile, and of the last (the tile
    // pass's workgroups' stretches of blocks, recorded by the bases pass)
    size_t tiles, flags, tgrp, total;
    uint64_t n_scan_blocks, scan_chunk, n_sel_blocks, max_tiles;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Scan grid for n entries: nb workgroups of `chunk` entries each (a multiple
// of kScanTile; the last one may be short), nb <= kMaxScanParts, none empty.
inline void scan_geom(uint64_t n, uint64_t *nb, uint64_t *chunk) {
    const uint64_t steps = (n + kScanTile - 1) / kScanTile;
    const uint64_t per = (steps + kMaxScanParts - 1) / kMaxScanParts;  // steps per workgroup
    *nb = per ? (steps + per - 1) / per : 0;
    *chunk = (per ? per : 1) * kScanTile;
}

inline WsLayout ws_fixed(uint64_t n) {
    WsLayout L{};
    scan_geom(n, &L.n_scan_blocks, &L.scan_chunk);
    constexpr uint64_t nb = kMaxScanParts;  // fixed: see kMaxScanParts
    size_t at = 0;
    L.header = at;    at += align256(sizeof(WsHeader));
    L.post = at;      at += align256(sizeof(WsHeader));  // statistics passes' own header
    L.part = at;      at += align256(nb * sizeof(ScanPart));
    L.spart = at;     at += align256(nb * sizeof(StatPart));
    L.csum = at;      at += align256(nb * 16 * sizeof(uint64_t));  // one-launch statistics
    // -- everything below here is a plan's: statistics passes stop above --
    L.tpart = at;     at += align256(2 * nb * sizeof(uint64_t));   // per tile-size candidate
    L.twhole = at;    at += align256(2 * nb * sizeof(uint64_t));
    L.lbase = at;     at += align256((nb + 1) * sizeof(uint64_t));
    L.live_dst = at;  at += align256((n + 1) * sizeof(uint64_t));
    L.live_src = at;  at += align256((n + 1) * sizeof(uint64_t));
    L.live_size = at; at += align256((n + 1) * sizeof(uint64_t));
    L.live_pin = at;  at += align256((n + 1) * sizeof(uint8_t));
    L.tile_base = at; at += align256((n + 1) * sizeof(uint32_t));
    L.n_sel_blocks = (n + 1 + kSelThreads - 1) / kSelThreads;
    L.live_z = at;    at += align256((n + 1) * sizeof(uint64_t));
    L.live_pc = at;   at += align256((n + 1) * sizeof(uint32_t));
    L.selpart = at;   at += align256(L.n_sel_blocks * sizeof(SelPart));
    L.live_rec = at;  at += align256((n + 1) * sizeof(LiveRec));
    L.live_key = at;  at += align256((n + 1) * sizeof(uint32_t));
    L.ridx = at;      at += align256((remap_bucket_cap(n) + 2) * sizeof(uint32_t));
    L.fixed = at;
    return L;
}

inline WsLayout ws_with_tiles(uint64_t n, uint64_t max_tiles) {
    WsLayout L = ws_fixed(n);
    L.max_tiles = max_tiles;
    size_t at = L.fixed;
    L.tiles = at;      at += align256(max_tiles * sizeof(TileRec));
    L.flags = at;      at += align256(max_tiles * sizeof(uint32_t));
    L.tgrp = at;       at += align256((max_tiles / 256 + 2) * sizeof(uint32_t));
    L.total = at;
    return L;
}

// Tiles a compaction may need: every window of the arena, plus the two
// partial windows at each end of every run of moved blocks (one run per
// segment at most, and there are max_pinned + 1 segments).
inline uint64_t tiles_bound(uint64_t arena_bytes, uint64_t max_pinned, uint32_t tile_bytes) {
    return arena_bytes / tile_bytes + 2 * (max_pinned + 1) + 2;
}

// The largest tile capacity whose layout fits in ws_bytes.
inline uint64_t tiles_fitting(uint64_t n, size_t ws_bytes) {
    const WsLayout F = ws_fixed(n);
    if (ws_bytes <= F.fixed) return 0;
    // upper estimate (each tile's record and flag and a 256th of a group
    // entry), then step down past the (at most 3 x 255 bytes of) alignment
    // padding and the two spare group entries: a few steps
    uint64_t t = (uint64_t)(ws_bytes - F.fixed) * 256 / (kPerTileBytes * 256 + sizeof(uint32_t));
    while (t > 0 && ws_with_tiles(n, t).total > ws_bytes) --t;
    return t;
}

// Table pointers as the kernels see them.
struct TableView {
    const uint64_t *off;
    const uint64_t *size;
    const uint8_t *live;    // may be null: all live
    const uint8_t *pinned;  // may be null: none pinned
    uint64_t n;             // entries
};

// Whether the plan whose header this is failed: an invalid table, no window
// for a targeted request, or more tiles than the workspace holds.
// (Every field is loaded before any is tested: one memory round trip, not
// one per field.)
__device__ inline bool plan_failed(const WsHeader *h, uint64_t max_tiles) {
    const uint64_t bad = h->bad_key, win = h->win_state, nt = h->n_tiles;
    return (bad != kNone) | (win == kWinNoFit) | (nt > max_tiles);
}

// Packed live-block arrays (m + 1 entries each).
struct LiveView {
    const uint64_t *dst;   // new offset
    const uint64_t *src;   // old offset
    const uint64_t *size;
    const uint8_t *pin;
};

inline LiveView live_view(const uint8_t *ws, const WsLayout &L) {
    return LiveView{reinterpret_cast<const uint64_t *>(ws + L.live_dst),
                    reinterpret_cast<const uint64_t *>(ws + L.live_src),
                    reinterpret_cast<const uint64_t *>(ws + L.live_size),
                    reinterpret_cast<const uint8_t *>(ws + L.live_pin)};
}

// Return the first failing step: a kernel launch reports through the
// thread's last-error state, so it is read after every launch, before a
// later launch can replace it.
#define AC_TRY(expr)                                    \
    do {                                                \
        const hipError_t ac_err_ = (expr);              \
        if (ac_err_ != hipSuccess) return ac_err_;      \
    } while (0)

// ---- plan.hip ----
// Plan and selection scans and, with kOutNew, the mover's tiles (for at most
// L.max_tiles tiles).  All asynchronous; the header then holds totals,
// statistics and n_tiles (tiles are built only if n_tiles <= L.max_tiles).
// fit_need: a hole size to first-fit (header fit_offset), kNone for none.
// clear: a word a plan's last scan pass sets to zero (the one-call path's
// invalid-handle count, so that its remap needs no launch of its own for
// it), or null.  A plan also clears the statistics header's count of
// finished workgroups, which launch_stats_one needs cleared.
hipError_t launch_scan(const TableView &t, uint64_t arena_bytes, uint8_t *ws,
                       const WsLayout &L, uint64_t *new_offset, int outputs,
                       TileChoice tiles, uint64_t epoch, uint64_t fit_need, uint64_t *clear,
                       hipStream_t s);
// Targeted plan: a selection scan, the window search (header win_*), then
// the plan scan with every live block outside the window held in place.
// Nothing is planned (and new_offset is not written) when no window fits.
hipError_t launch_targeted(const TableView &t, uint64_t arena_bytes, uint64_t request,
                           uint8_t *ws, const WsLayout &L, uint64_t *new_offset,
                           TileChoice tiles, uint64_t epoch, uint64_t *clear, hipStream_t s);
// A statistics pass (and, if fit_need != kNone, the first fit) in one
// launch, into the header at L.header.  Its last workgroup finds itself by
// a count in that header: after_plan -- a plan ran on this workspace
// before, in stream order, and cleared it (each pass leaves it cleared) --
// or else a one-thread launch clears it first.
hipError_t launch_stats_one(const TableView &t, uint64_t arena_bytes, uint8_t *ws,
                            const WsLayout &L, uint64_t fit_need, bool after_plan,
                            hipStream_t s);
// A read-back's device half: words 8-byte words from src (device) into
// dst_host (pinned, device-mapped host memory), then seq into *seq_host.
hipError_t launch_publish(const uint64_t *src, uint64_t *dst_host, uint32_t words,
                          uint64_t *seq_host, uint64_t seq, hipStream_t s);

// Copy `bytes` (a positive multiple of 8, at most 1 KiB) of device memory
// into host memory, queued on s behind everything queued before, and wait
// for it: DEFRAG_OK, DEFRAG_EHIP (a HIP call or a queued kernel failed) or
// DEFRAG_EINVAL (a size outside those bounds).
int read_back(void *out_host, const void *src_dev, uint32_t bytes, hipStream_t s);

// While one lives, the calling thread's read-backs allocate nothing: they
// copy into the caller's pageable memory.
struct NoAllocScope {
    NoAllocScope();
    ~NoAllocScope();
    NoAllocScope(const NoAllocScope &) = delete;
    NoAllocScope &operator=(const NoAllocScope &) = delete;
};

hipError_t launch_commit(const uint8_t *ws, const WsLayout &L, uint64_t live_blocks,
                         uint64_t *off_out, uint64_t *size_out, uint8_t *live_out,
                         uint8_t *pinned_out, hipStream_t s);

// ---- move.hip ----
struct MoveArgs {
    uint8_t *arena;
    const uint64_t *live_dst;  // new offset of every live block
    const uint64_t *live_src;  // old offset of every live block
    const TileRec *tiles;
    uint32_t *flags;
    WsHeader *hdr;
    uint64_t n_tiles;
    uint64_t epoch;
    uint64_t spin_limit;
    uint32_t tile_bytes;
    uint32_t max_blocks;  // LDS capacity in block descriptors
    uint32_t small_blocks;  // launch kMoveThreadsSmallBlocks lanes per workgroup
    // Sized on the device: the mover is queued right behind its plan, before
    // the host has read the plan back, so the tile count and the workgroups
    // that take part come from the header, and a failed plan moves nothing.
    uint32_t device_sized;
    uint32_t wg_per_cu;   // device-sized: 0 = the default (kDefaultWgPerCu)
    uint32_t num_cus;
    uint64_t max_tiles;   // device-sized: the workspace's tile capacity
    // What the check pass before a separate move holds each tile record to
    // (a workspace overwritten since its plan moves nothing: kStatusCorrupt).
    uint64_t arena_bytes;
    uint64_t live_blocks; // entries of the packed live arrays
    // Wait-path testing knob (0 = off): tile t holds its "sources read" flag
    // back for stall_sleeps sleeps when mix(t, stall_seed) % stall_every == 0.
    uint32_t stall_every;
    uint32_t stall_sleeps;
    uint32_t stall_seed;
    uint32_t pad;
};
hipError_t launch_move(const MoveArgs &a, uint32_t wg_per_cu, uint32_t nontemporal,
                       int num_cus, hipStream_t s);
// The device-sized mover: a grid for the largest workgroup count the rule
// can pick, and LDS for the most blocks a tile can meet.  side (or null):
// a side job (remap.hip, with a gate) that the launch's first workgroups
// run beside the move if the plan chose this mover's tile size or
// side->any_tile is set (of two movers, the chosen one's launch runs it).
struct SideArgs;
hipError_t launch_move_device_sized(const MoveArgs &a, uint32_t nontemporal,
                                    const SideArgs *side, hipStream_t s);

// ---- api.cpp ----
// The whole compaction in the plain order on one stream, creating nothing:
// defrag_compact's fallback, and the static-scratch entry point's body.
int compact_serial(const struct defrag_compact_args *a, hipStream_t stream,
                   struct defrag_plan_t *plan, struct defrag_stats_t *after_host);

// ---- remap.hip ----
// The packed table's outputs (defrag_commit's); a null pointer is not written.
struct CommitOut {
    uint64_t *off;
    uint64_t *size;
    uint8_t *live;
    uint8_t *pinned;
};
// The part of a compaction that reads the plan and never the arena, as one
// job for a range of workgroups (side.h): the handle remap (h_in -> h_out,
// H handles, those in no live block counted into n_invalid), the packed
// table (commit != 0: the plan's packed live arrays into out) and the
// post-check (post != 0: the statistics of that packed table into
// post_hdr, its chunk summaries in csum).  m: the live-block count, or with
// a gate (the plan's header, for a job queued before the plan is read
// back) the most there can be: the job then takes the header's count, and
// does nothing if the plan failed.
enum : uint32_t { kSideEnt = 0, kSideRec32 = 1, kSideRec64 = 2 };
struct SideArgs {
    const void *rec;           // RemapEnt, LiveRec32 or LiveRec records
    const uint64_t *live_src;  // old offsets (searched when key is null)
    const uint32_t *key;       // 32-bit keys, or null
    const uint32_t *ridx;      // bucket index
    uint64_t nb;               // buckets
    uint32_t w;                // log2 of the bucket width
    uint32_t kind;             // kSideEnt, kSideRec32 or kSideRec64
    const uint64_t *h_in;
    uint64_t *h_out;
    uint64_t H;
    unsigned long long *n_invalid;
    uint64_t m;
    const WsHeader *gate;
    uint64_t max_tiles;
    LiveView lv;
    CommitOut out;
    uint32_t commit;
    uint32_t post;
    uint64_t arena_bytes, chunk, ngroups;  // post-check: chunks of the packed table (size_side)
    void *csum;
    WsHeader *post_hdr;
    uint64_t work;      // the most entries or handles one lane pass covers
    uint32_t groups;    // workgroups running the job (set by the launch)
    uint32_t any_tile;  // in a mover's launch: run whatever tile size the plan chose
};
// A side job on the plan in the workspace (n: the planned table's entries;
// live_blocks: its live count, or the most there can be with a gate).
SideArgs side_args(const uint8_t *ws, const WsLayout &L, uint64_t arena_bytes, uint64_t n,
                   uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out,
                   uint64_t n_handles, uint64_t *n_invalid, const CommitOut *commit, bool post,
                   const WsHeader *gate, uint64_t max_tiles);
// Size a side job for workgroups of `lanes` lanes: enough workgroups for
// its work, at most 512 lanes per compute unit and kMaxScanParts (groups),
// and the post-check's chunks of the packed table, one per workgroup at
// most (chunk, ngroups).
void size_side(SideArgs &sj, uint32_t lanes, int num_cus);
// defrag_remap: the handle remap alone, in a launch of its own (n_invalid
// cleared first).
hipError_t launch_remap(const uint8_t *ws, const WsLayout &L, uint64_t arena_bytes, uint64_t n,
                        uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out,
                        uint64_t n_handles, uint64_t *n_invalid, int num_cus, hipStream_t s);

}  // namespace ac

#pragma GCC visibility pop

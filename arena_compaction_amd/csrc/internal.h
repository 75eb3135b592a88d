// internal.h -- workspace layout and kernel launchers shared by the library's
// own sources (api.cpp, plan.hip, move.hip, remap.hip).  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ac {

constexpr uint32_t kScanThreads = 256;          // threads per scan workgroup
constexpr uint32_t kScanItems = 8;              // table entries per thread
constexpr uint32_t kScanTile = kScanThreads * kScanItems;  // entries per workgroup
constexpr uint32_t kSpineThreads = 1024;        // single-workgroup passes
constexpr uint32_t kMoveThreads = 256;          // mover workgroup
constexpr uint32_t kMoveRowBytes = kMoveThreads * 16;  // one 16-B vector per lane
constexpr uint32_t kDefaultTile = 65536;
constexpr uint32_t kDefaultWgPerCu = 2;     // measured best on the 80 GiB workload
constexpr uint32_t kDefaultNontemporal = 1; // streaming loads and stores
constexpr uint32_t kMinTile = 256;
constexpr uint32_t kMaxTile = 131072;
constexpr uint32_t kDefaultSpinLog2 = 22;
constexpr uint64_t kNone = ~0ull;

// Device-resident plan header (first 256 bytes of the workspace).
struct alignas(256) WsHeader {
    uint64_t live_bytes;     // LT: sum of live sizes
    uint64_t live_blocks;    // m
    uint64_t max_live_end;   // end of the highest live block (0 if none)
    uint64_t bad_key;        // (index << 3) | reason of the first bad entry, kNone if valid
    uint64_t largest_hole;   // longest run outside live blocks, tail included
    uint64_t hole_count;     // number of such runs
    uint64_t moved_blocks;
    uint64_t moved_bytes;
    uint64_t first_moved;    // index (among live blocks) of the first moved block, m if none
    uint64_t min_live_size;  // kNone if no live block
    uint64_t move_begin;     // new offset of the first moved block (LT if none)
    uint64_t epoch;          // plan epoch, checked by the mover
    uint32_t ticket;         // mover tile ticket counter
    uint32_t status;         // mover status bits (kStatus*)
    uint64_t pad[19];
};
static_assert(sizeof(WsHeader) == 256, "header size");

constexpr uint32_t kStatusTimeout = 1u;  // a wait gave up, or a tile overflowed LDS

// Per scan-workgroup aggregate of (live size sum, live end max, live count)
// plus the smallest bad-entry key seen.
struct ScanPart {
    uint64_t sum;
    uint64_t maxend;
    uint64_t count;
    uint64_t bad_key;
};

// Per scan-workgroup hole / move statistics.
struct StatPart {
    uint64_t max_gap;
    uint64_t gaps;
    uint64_t moved_blocks;
    uint64_t moved_bytes;
    uint64_t first_moved;
    uint64_t min_size;
    uint64_t pad[2];
};

// Per destination tile: live-block range touching it and the earlier tiles
// whose sources overlap it (dep_lo > dep_hi means none).
struct TileRec {
    uint32_t first_block;
    uint32_t last_block;
    uint32_t dep_lo;
    uint32_t dep_hi;
};

struct WsLayout {
    size_t header, part, prefix, spart, live_dst, live_src, tiles, flags, total;
    uint64_t n_scan_blocks, max_tiles;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(uint64_t n, uint64_t arena_bytes, uint32_t tile_bytes) {
    WsLayout L{};
    L.n_scan_blocks = (n + kScanTile - 1) / kScanTile;
    uint64_t nb = L.n_scan_blocks ? L.n_scan_blocks : 1;
    L.max_tiles = arena_bytes / tile_bytes + 2;
    size_t at = 0;
    L.header = at;   at += align256(sizeof(WsHeader));
    L.part = at;     at += align256(nb * sizeof(ScanPart));
    L.prefix = at;   at += align256(nb * sizeof(ScanPart));
    L.spart = at;    at += align256(nb * sizeof(StatPart));
    L.live_dst = at; at += align256((n + 1) * sizeof(uint64_t));
    L.live_src = at; at += align256((n + 1) * sizeof(uint64_t));
    L.tiles = at;    at += align256(L.max_tiles * sizeof(TileRec));
    L.flags = at;    at += align256(L.max_tiles * sizeof(uint32_t));
    L.total = at;
    return L;
}

// Table pointers as the kernels see them.
struct TableView {
    const uint64_t *off;
    const uint64_t *size;
    const uint8_t *live;  // may be null: all live
    uint64_t n;
};

// ---- plan.hip ----
hipError_t launch_scan(const TableView &t, uint64_t arena_bytes, uint8_t *ws,
                       const WsLayout &L, uint64_t *new_offset, bool write_outputs,
                       uint64_t epoch, hipStream_t s);
hipError_t launch_tiles(uint8_t *ws, const WsLayout &L, uint64_t n_tiles,
                        uint64_t tile_base, uint32_t tile_bytes, uint64_t move_begin,
                        uint64_t live_bytes, uint64_t first_moved, uint64_t live_blocks,
                        hipStream_t s);
hipError_t launch_commit(const uint8_t *ws, const WsLayout &L, uint64_t live_blocks,
                         uint64_t *off_out, uint64_t *size_out, uint8_t *live_out,
                         hipStream_t s);

// ---- move.hip ----
struct MoveArgs {
    uint8_t *arena;
    const uint64_t *live_dst;  // new offset of every live block, [m] = LT
    const uint64_t *live_src;  // old offset of every live block
    const TileRec *tiles;
    uint32_t *flags;
    WsHeader *hdr;
    uint64_t n_tiles;
    uint64_t tile_base;
    uint64_t move_begin;
    uint64_t live_bytes;
    uint64_t epoch;
    uint64_t spin_limit;
    uint32_t tile_bytes;
    uint32_t max_blocks;  // LDS capacity in block descriptors
};
hipError_t launch_move(const MoveArgs &a, uint32_t wg_per_cu, uint32_t nontemporal,
                       int num_cus, hipStream_t s);

// ---- remap.hip ----
hipError_t launch_remap(const uint64_t *live_dst, const uint64_t *live_src,
                        uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out,
                        uint64_t n_handles, uint64_t *n_invalid, int num_cus,
                        hipStream_t s);

}  // namespace ac

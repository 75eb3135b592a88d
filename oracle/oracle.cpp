// oracle.cpp -- plain single-threaded CPU oracle for in-place arena compaction.
//
// TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  It
// shares nothing with the HIP library.  Each function states the passage of
// the pages it writes out; see oracle.h for the page titles.
//
// Readings where the pages are silent:
//  * a hole is any maximal byte run not covered by a live entry -- free
//    entries, untracked gaps and the tail alike; adjacent free pieces form one
//    hole, as the CANN pool merges adjacent free blocks ([CANN] 2.2);
//  * entries are 32-byte aligned and non-empty ([CANN] 2.2 rounds every
//    request up to 32 bytes; 3.3 aligns allocations to 32 or 64 bytes);
//  * compaction keeps block order and packs each segment from its start with
//    no padding: every movable live block moves down by the total hole size
//    below it in its segment ([910C] periodic compaction: holes scanned low to
//    high, downward shift); with nothing pinned the one segment starts at 0;
//  * a pinned block ([910C] fixed-address parameter region) is live and stays;
//  * bytes that no movable block lands on keep whatever they held.
#include "oracle.h"

#include <algorithm>
#include <cstring>
#include <vector>

namespace {

inline bool is_pinned(const uint8_t *pinned, uint64_t i) { return pinned && pinned[i]; }

}  // namespace

extern "C" {

// Entry checks, lowest entry first; within an entry the checks run in the
// order documented in oracle.h.
int oracle_validate(const uint64_t *offset, const uint64_t *size,
                    const uint8_t *live, const uint8_t *pinned, uint64_t n,
                    uint64_t arena_bytes, uint64_t *bad_index, int32_t *reason) {
    *bad_index = UINT64_MAX;
    *reason = ORACLE_REASON_NONE;
    for (uint64_t i = 0; i < n; ++i) {
        int32_t r = ORACLE_REASON_NONE;
        if (size[i] == 0)
            r = ORACLE_REASON_ZERO_SIZE;
        else if (offset[i] % 32 != 0 || size[i] % 32 != 0)
            r = ORACLE_REASON_MISALIGNED;
        else if (live[i] > 1)
            r = ORACLE_REASON_LIVE_FLAG;
        else if (pinned && (pinned[i] > 1 || (pinned[i] == 1 && live[i] == 0)))
            r = ORACLE_REASON_PINNED_FLAG;
        else if (offset[i] > arena_bytes || size[i] > arena_bytes - offset[i])
            r = ORACLE_REASON_OUT_OF_ARENA;
        else if (i > 0 && offset[i - 1] + size[i - 1] > offset[i])
            r = ORACLE_REASON_OVERLAP;
        if (r != ORACLE_REASON_NONE) {
            *bad_index = i;
            *reason = r;
            return ORACLE_EINVAL;
        }
    }
    return ORACLE_OK;
}

// [910C] periodic compaction: each live tensor moves toward low addresses by
// the holes below it, so its new start is its segment's start plus the live
// data below it in the segment.  A pinned block stays and starts a segment.
void oracle_new_offsets(const uint64_t *offset, const uint64_t *size,
                        const uint8_t *live, const uint8_t *pinned, uint64_t n,
                        uint64_t *new_offset) {
    uint64_t running = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (is_pinned(pinned, i)) {
            new_offset[i] = offset[i];
            running = offset[i] + size[i];
            continue;
        }
        new_offset[i] = running;
        if (live[i]) running += size[i];
    }
}

// [910C] periodic compaction, "move the data"; [CANN] 3.3 periodic
// compaction gathers every allocated block into one contiguous region.
// Lowest block first: block i's destination lies in its own segment and can
// only overlap its own source (memmove copes) and sources of lower blocks,
// which have already moved.
void oracle_compact(uint8_t *arena, uint64_t arena_bytes,
                    const uint64_t *offset, const uint64_t *size,
                    const uint8_t *live, const uint8_t *pinned, uint64_t n) {
    (void)arena_bytes;
    uint64_t dst = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (is_pinned(pinned, i)) {
            dst = offset[i] + size[i];
            continue;
        }
        if (!live[i]) continue;
        if (dst != offset[i])
            std::memmove(arena + dst, arena + offset[i], size[i]);
        dst += size[i];
    }
}

// [910C] monitoring: the free total and the largest contiguous free block,
// and free/largest - 1.  [CANN] 3.2: 1 - largest/free, 0 when nothing is
// free (the same rule is taken for the first ratio).  [CANN] 2.2: adjacent
// free blocks merge, so a hole is the whole gap between two live blocks.
void oracle_stats_walk(const uint64_t *offset, const uint64_t *size,
                       const uint8_t *live, const uint8_t *pinned, uint64_t n,
                       uint64_t arena_bytes, oracle_stats *out) {
    std::memset(out, 0, sizeof(*out));
    out->arena_bytes = arena_bytes;
    uint64_t cursor = 0;   // end of the last live block seen so far
    uint64_t new_off = 0;  // where the current movable block would land
    for (uint64_t i = 0; i < n; ++i) {
        if (!live[i]) continue;
        const uint64_t gap = offset[i] - cursor;
        if (gap > 0) {
            out->hole_count += 1;
            if (gap > out->largest_hole) out->largest_hole = gap;
        }
        out->live_blocks += 1;
        out->live_bytes += size[i];
        if (is_pinned(pinned, i)) {
            new_off = offset[i] + size[i];
        } else {
            if (offset[i] != new_off) {
                out->moved_blocks += 1;
                out->moved_bytes += size[i];
            }
            new_off += size[i];
        }
        cursor = offset[i] + size[i];
    }
    const uint64_t tail = arena_bytes - cursor;
    if (tail > 0) {
        out->hole_count += 1;
        if (tail > out->largest_hole) out->largest_hole = tail;
    }
    out->free_bytes = arena_bytes - out->live_bytes;
    if (out->free_bytes == 0) {
        out->frag_free_over_largest_minus_1 = 0.0;
        out->frag_one_minus_largest_over_free = 0.0;
    } else {
        const double F = (double)out->free_bytes;
        const double L = (double)out->largest_hole;
        out->frag_free_over_largest_minus_1 = F / L - 1.0;
        out->frag_one_minus_largest_over_free = 1.0 - L / F;
    }
}

// [910C] periodic compaction, "update the references in one batch"; and
// "Moving to other accelerators": without a framework call that rewrites
// tensor addresses, references are kept at operator level -- here a handle is
// a byte address in the arena; it keeps its offset inside its block.
void oracle_remap(const uint64_t *offset, const uint64_t *size,
                  const uint8_t *live, const uint8_t *pinned, uint64_t n,
                  const uint64_t *h_in, uint64_t *h_out, uint64_t n_handles,
                  uint64_t *n_invalid) {
    std::vector<uint64_t> new_off(n);
    oracle_new_offsets(offset, size, live, pinned, n, new_off.data());
    uint64_t bad = 0;
    for (uint64_t k = 0; k < n_handles; ++k) {
        const uint64_t h = h_in[k];
        const uint64_t *it = std::upper_bound(offset, offset + n, h);
        uint64_t result = UINT64_MAX;
        if (it != offset) {
            const uint64_t i = (uint64_t)(it - offset) - 1;
            if (live[i] && h - offset[i] < size[i])
                result = new_off[i] + (h - offset[i]);
        }
        if (result == UINT64_MAX) bad += 1;
        h_out[k] = result;
    }
    *n_invalid = bad;
}

// The compacted arena written as a function of the original one: a byte a
// movable live block lands on holds that block's byte at the same offset
// inside the block; every other byte is untouched.
int64_t oracle_source_map(const uint64_t *offset, const uint64_t *size,
                          const uint8_t *live, const uint8_t *pinned, uint64_t n,
                          uint64_t arena_bytes, uint64_t p0, uint64_t len,
                          uint64_t *seg_dst, uint64_t *seg_src, uint64_t *seg_len,
                          uint64_t cap) {
    (void)arena_bytes;
    const uint64_t p1 = p0 + len;
    uint64_t count = 0;
    uint64_t covered = p0;  // window bytes below this are already emitted
    auto emit = [&](uint64_t d, uint64_t s, uint64_t l) -> bool {
        if (count == cap) return false;
        seg_dst[count] = d;
        seg_src[count] = s;
        seg_len[count] = l;
        ++count;
        return true;
    };
    uint64_t dst = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (is_pinned(pinned, i)) {
            dst = offset[i] + size[i];
            continue;
        }
        if (!live[i]) continue;
        const uint64_t a = std::max(dst, p0);
        const uint64_t b = std::min(dst + size[i], p1);
        if (a < b) {
            if (covered < a && !emit(covered, covered, a - covered)) return -1;
            if (!emit(a, offset[i] + (a - dst), b - a)) return -1;
            covered = b;
        }
        dst += size[i];
    }
    if (covered < p1 && !emit(covered, covered, p1 - covered)) return -1;
    return (int64_t)count;
}

// [910C] "Periodic compaction with Ascend C": compaction pauses every tensor
// it touches, so it is a stop-loss step, and the failure it answers is one
// request (the 4.2 GB communication buffer) larger than any free block.
// Holes are listed low to high; between two neighbouring holes lie some live
// bytes, and possibly a pinned block, which no window may contain.  A sweep
// over the last hole of the window keeps, for each, the shortest window
// ending there that still frees `request` bytes (its first hole only moves
// up as the last one does), and the cheapest of those wins.
int oracle_target_window(const uint64_t *offset, const uint64_t *size,
                         const uint8_t *live, const uint8_t *pinned, uint64_t n,
                         uint64_t arena_bytes, uint64_t request, oracle_window *out) {
    std::memset(out, 0, sizeof(*out));
    if (request == 0) return ORACLE_EINVAL;
    struct Hole {
        uint64_t start, len;
        uint64_t live_after;  // live bytes between this hole and the next
        bool pinned_after;    // a pinned block lies between them
    };
    std::vector<Hole> holes;
    uint64_t cursor = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (!live[i]) continue;
        if (offset[i] > cursor) holes.push_back(Hole{cursor, offset[i] - cursor, 0, false});
        if (!holes.empty()) {
            holes.back().live_after += size[i];
            if (is_pinned(pinned, i)) holes.back().pinned_after = true;
        }
        cursor = offset[i] + size[i];
    }
    if (arena_bytes > cursor) holes.push_back(Hole{cursor, arena_bytes - cursor, 0, false});

    uint64_t first = 0, free_sum = 0, live_sum = 0;
    for (uint64_t last = 0; last < holes.size(); ++last) {
        if (last > 0) {
            if (holes[last - 1].pinned_after) {  // start again past the barrier
                first = last;
                free_sum = 0;
                live_sum = 0;
            } else {
                live_sum += holes[last - 1].live_after;
            }
        }
        free_sum += holes[last].len;
        while (first < last && free_sum - holes[first].len >= request) {
            free_sum -= holes[first].len;
            live_sum -= holes[first].live_after;
            ++first;
        }
        if (free_sum < request) continue;
        const uint64_t begin = holes[first].start;
        if (!out->found || live_sum < out->moved_bytes ||
            (live_sum == out->moved_bytes && begin < out->begin)) {
            out->found = 1;
            out->begin = begin;
            out->end = holes[last].start + holes[last].len;
            out->hole = free_sum;
            out->moved_bytes = live_sum;
        }
    }
    return ORACLE_OK;
}

// [CANN] 2.2: the pool rounds a request up to 32 bytes and takes the first
// free block that holds it; adjacent free blocks are merged, so a free block
// is a whole hole.  Walk the holes from low to high addresses.
int oracle_first_fit(const uint64_t *offset, const uint64_t *size,
                     const uint8_t *live, uint64_t n, uint64_t arena_bytes,
                     uint64_t request, uint64_t *offset_out) {
    *offset_out = UINT64_MAX;
    if (request == 0 || request > UINT64_MAX - 31) return ORACLE_EINVAL;
    const uint64_t need = (request + 31) / 32 * 32;
    uint64_t cursor = 0;  // end of the last live block
    for (uint64_t i = 0; i < n; ++i) {
        if (!live[i]) continue;
        if (offset[i] - cursor >= need) {
            *offset_out = cursor;
            return ORACLE_OK;
        }
        cursor = offset[i] + size[i];
    }
    if (arena_bytes - cursor >= need) *offset_out = cursor;
    return ORACLE_OK;
}

// [CANN] 5.3 MemoryMonitor.check / predict_oom_time, and the 910C page's
// rule of reading the largest free block next to the free total.
void oracle_monitor(uint64_t arena_bytes, uint64_t live_bytes, uint64_t largest_hole,
                    double warning_ratio, double critical_ratio, double frag_threshold,
                    uint64_t next_request, double growth_bytes_per_s,
                    oracle_monitor_out *out) {
    std::memset(out, 0, sizeof(*out));
    const uint64_t free_bytes = arena_bytes - live_bytes;
    const double usage = arena_bytes ? (double)live_bytes / (double)arena_bytes : 0.0;
    out->usage_ratio = usage;
    if (usage > critical_ratio)
        out->level = ORACLE_LEVEL_CRITICAL;
    else if (usage > warning_ratio)
        out->level = ORACLE_LEVEL_WARNING;
    else
        out->level = ORACLE_LEVEL_OK;
    out->frag_free_over_largest_minus_1 =
        free_bytes ? (double)free_bytes / (double)largest_hole - 1.0 : 0.0;
    out->seconds_to_full = growth_bytes_per_s > 0.0
                               ? (double)free_bytes / growth_bytes_per_s
                               : __builtin_inf();
    out->action = ORACLE_ACTION_NONE;
    if (next_request > 0) {
        // a request past 2^64 - 32 rounds to something no arena holds
        const bool huge = next_request > UINT64_MAX - 31;
        const uint64_t need = huge ? UINT64_MAX : (next_request + 31) / 32 * 32;
        if (huge || need > largest_hole) {
            out->action = (!huge && need <= free_bytes) ? ORACLE_ACTION_TARGETED
                                                        : ORACLE_ACTION_NO_ROOM;
            return;
        }
    }
    if (frag_threshold > 0.0 && out->frag_free_over_largest_minus_1 > frag_threshold)
        out->action = ORACLE_ACTION_FULL;
}

}  // extern "C"

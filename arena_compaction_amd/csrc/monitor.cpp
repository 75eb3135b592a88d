// monitor.cpp -- the layout monitor: host arithmetic on statistics that
// defrag_stats measured on the device.  No HIP call.
//
// Page "CANN memory management and memory optimisation", section 5.3
// (MemoryMonitor): usage = used / total is rated against a warning and a
// critical ratio, an alarm being raised when a ratio is exceeded, and the
// time until the memory is full is the remaining bytes over the growth rate
// (never, for a rate that is not positive).  Page "Ascend 910C cluster
// tuning": the free total alone hides fragmentation (section "Total-usage
// monitoring misses fragmentation"); when an allocation fails with enough
// memory free, the layout and not the capacity is at fault (closing
// advice); compaction pauses what it touches and is kept for stopping the
// damage (section "Periodic compaction with Ascend C").  So: a pending
// request the largest hole cannot hold -- after the CANN pool's rounding to
// 32 bytes, section 2.2 -- asks for a targeted compaction if the free total
// could hold it and for capacity if not; otherwise a fragmentation ratio
// above the caller's threshold asks for a full compaction.
#include <cmath>
#include <cstring>

#include "../../include/arena_compaction.h"

extern "C" int defrag_monitor(const defrag_stats_t *stats, const defrag_monitor_cfg *cfg,
                              defrag_monitor_report *out) {
    if (!stats || !out) return DEFRAG_EINVAL;
    std::memset(out, 0, sizeof(*out));
    defrag_monitor_cfg c{0.85, 0.95, 0.0, 0, 0.0};
    if (cfg) c = *cfg;
    if (stats->invalid_reason != DEFRAG_REASON_NONE) return DEFRAG_EINVAL;
    if (std::isnan(c.warning_ratio) || std::isnan(c.critical_ratio) ||
        std::isnan(c.frag_threshold) || std::isnan(c.growth_bytes_per_s))
        return DEFRAG_EINVAL;
    const uint64_t total = stats->arena_bytes;
    const uint64_t used = stats->live_bytes;
    const uint64_t avail = stats->free_bytes;
    if (used > total || avail != total - used || stats->largest_hole > avail)
        return DEFRAG_EINVAL;

    out->usage_ratio = total ? static_cast<double>(used) / static_cast<double>(total) : 0.0;
    out->level = out->usage_ratio > c.critical_ratio  ? DEFRAG_LEVEL_CRITICAL
                 : out->usage_ratio > c.warning_ratio ? DEFRAG_LEVEL_WARNING
                                                      : DEFRAG_LEVEL_OK;
    out->frag_free_over_largest_minus_1 = stats->frag_free_over_largest_minus_1;
    out->frag_one_minus_largest_over_free = stats->frag_one_minus_largest_over_free;
    out->seconds_to_full = c.growth_bytes_per_s > 0.0
                               ? static_cast<double>(avail) / c.growth_bytes_per_s
                               : HUGE_VAL;

    out->action = DEFRAG_ACTION_NONE;
    if (c.next_request) {
        // the pool places ceil32(request) bytes; past 2^64 - 32 nothing fits
        const bool fits_u64 = c.next_request <= UINT64_MAX - 31;
        const uint64_t placed = fits_u64 ? ((c.next_request + 31) & ~uint64_t(31)) : UINT64_MAX;
        if (!fits_u64 || placed > stats->largest_hole) {
            out->action = (fits_u64 && placed <= avail) ? DEFRAG_ACTION_TARGETED
                                                        : DEFRAG_ACTION_NO_ROOM;
            return DEFRAG_OK;
        }
    }
    if (c.frag_threshold > 0.0 && out->frag_free_over_largest_minus_1 > c.frag_threshold)
        out->action = DEFRAG_ACTION_FULL;
    return DEFRAG_OK;
}

/*
 * oracle.h -- plain, single-threaded CPU oracle for in-place arena compaction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; the two agree only because both follow the same pages.
 *
 * Pages followed (cited by title and section):
 *   [910C]  "Ascend 910C cluster tuning: memory-fragment compaction in
 *           mixed-precision training" -- sections "Total-usage monitoring
 *           misses fragmentation" (free total, largest contiguous free block,
 *           ratio free/largest - 1) and "Periodic compaction with Ascend C"
 *           (mark live tensors; scan holes from low to high addresses and give
 *           every live tensor its downward shift; move, then update every
 *           reference in one batch).
 *   [CANN]  "CANN memory management and memory optimisation: the NPU storage
 *           hierarchy" -- section 2.2 (memory pool: 32-byte rounding, adjacent
 *           free blocks merge into one), section 3.2 (fragmentation rate
 *           1 - largest/free, defined as 0 when nothing is free) and section
 *           3.3 (periodic compaction moves every allocated block into one
 *           contiguous region, leaving one large free region).
 *   [910C] section "Cutting alloc and free at the source": the parameter
 *           region keeps fixed addresses and is never freed.  A pinned entry
 *           models such a block: it is live, never moves, and splits the
 *           arena into segments that compact independently.
 *
 * All byte quantities are unsigned 64-bit.  The table is structure-of-arrays:
 * offset[n], size[n], live[n] (0/1) and pinned[n] (0/1, or NULL: nothing
 * pinned), host memory, owned by the caller.
 *
 * Segments: a segment is the span between two consecutive pinned blocks (or
 * an arena end).  Within each segment the movable live blocks keep their
 * order and pack down to the segment's start; pinned blocks stay put.  With
 * nothing pinned there is one segment, [0, arena_bytes).
 */
#ifndef ARENA_COMPACTION_ORACLE_H
#define ARENA_COMPACTION_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* Which check rejected a table entry: the first failing entry, and within it
 * the first failing check in the order zero size, misaligned, live flag,
 * pinned flag, out of arena, overlap. */
#define ORACLE_REASON_NONE 0
#define ORACLE_REASON_ZERO_SIZE 1      /* size == 0                          */
#define ORACLE_REASON_MISALIGNED 2     /* offset or size not a multiple of 32 */
#define ORACLE_REASON_LIVE_FLAG 3      /* live not 0 or 1                     */
#define ORACLE_REASON_OUT_OF_ARENA 4   /* offset + size > arena bytes         */
#define ORACLE_REASON_OVERLAP 5        /* starts before the previous one ends */
#define ORACLE_REASON_PINNED_FLAG 7    /* pinned not 0/1, or pinned but free  */

typedef struct oracle_stats {
    uint64_t arena_bytes;
    uint64_t live_bytes;
    uint64_t free_bytes;
    uint64_t largest_hole;
    uint64_t hole_count;
    uint64_t live_blocks;
    uint64_t moved_blocks;
    uint64_t moved_bytes;
    double frag_free_over_largest_minus_1;   /* [910C] monitoring section */
    double frag_one_minus_largest_over_free; /* [CANN] section 3.2        */
} oracle_stats;

/* Validate a table; on failure set *bad_index and *reason. */
int oracle_validate(const uint64_t *offset, const uint64_t *size,
                    const uint8_t *live, const uint8_t *pinned, uint64_t n,
                    uint64_t arena_bytes, uint64_t *bad_index, int32_t *reason);

/* new_offset[i]: a pinned entry keeps its offset; any other entry gets its
 * segment's start plus the sizes of the movable live entries before it in
 * that segment (with nothing pinned: the live bytes before it). */
void oracle_new_offsets(const uint64_t *offset, const uint64_t *size,
                        const uint8_t *live, const uint8_t *pinned, uint64_t n,
                        uint64_t *new_offset);

/* Ordered in-place compaction of a host arena: movable live blocks, lowest
 * first, memmove'd to their new offsets. */
void oracle_compact(uint8_t *arena, uint64_t arena_bytes,
                    const uint64_t *offset, const uint64_t *size,
                    const uint8_t *live, const uint8_t *pinned, uint64_t n);

/* Free total, holes and ratios by one low-to-high walk. */
void oracle_stats_walk(const uint64_t *offset, const uint64_t *size,
                       const uint8_t *live, const uint8_t *pinned, uint64_t n,
                       uint64_t arena_bytes, oracle_stats *out);

/* Address of every handle after compaction, UINT64_MAX if the handle is not
 * inside a live block; *n_invalid counts the latter.  h_out may equal h_in. */
void oracle_remap(const uint64_t *offset, const uint64_t *size,
                  const uint8_t *live, const uint8_t *pinned, uint64_t n,
                  const uint64_t *h_in, uint64_t *h_out, uint64_t n_handles,
                  uint64_t *n_invalid);

/* Where each byte of the compacted arena window [p0, p0+len) came from in the
 * original arena, as pieces (dst, src, len), ascending.  Returns the number
 * of pieces, or -1 if more than cap are needed.  A byte that no movable live
 * block lands on (pinned bytes, each segment's top hole) keeps its original
 * value, so its src equals its dst. */
int64_t oracle_source_map(const uint64_t *offset, const uint64_t *size,
                          const uint8_t *live, const uint8_t *pinned, uint64_t n,
                          uint64_t arena_bytes, uint64_t p0, uint64_t len,
                          uint64_t *seg_dst, uint64_t *seg_src, uint64_t *seg_len,
                          uint64_t cap);

/* Targeted compaction ([910C] periodic compaction is a costly global pause,
 * kept for stopping the damage; the failure it answers is one request -- the
 * 4.2 GB communication buffer -- that no contiguous free block can hold).
 * A window is a run of consecutive holes together with the live blocks
 * between them, none of them pinned.  Packing the window's blocks down to
 * the window's start (the other blocks stay) merges its holes into one at
 * the window's top.  The chosen window is the one whose merged hole holds at
 * least `request` bytes with the fewest live bytes inside (the bytes that
 * move); among those, the one starting lowest. */
typedef struct oracle_window {
    uint64_t found;        /* 0: no window can hold the request              */
    uint64_t begin;        /* window = [begin, end): from its first hole's   */
    uint64_t end;          /*   start to its last hole's end                 */
    uint64_t hole;         /* free bytes inside = the merged hole's size     */
    uint64_t moved_bytes;  /* live bytes inside                              */
} oracle_window;

/* Returns ORACLE_EINVAL for request == 0, else ORACLE_OK.  The table must
 * be valid (oracle_validate). */
int oracle_target_window(const uint64_t *offset, const uint64_t *size,
                         const uint8_t *live, const uint8_t *pinned, uint64_t n,
                         uint64_t arena_bytes, uint64_t request, oracle_window *out);

/* First fit ([CANN] 2.2 memory pool): a request is rounded up to a multiple
 * of 32 bytes and placed at the start of the first free block, in the
 * pool's merged free list, that can hold it.  Here the merged free list is
 * the table's holes in address order, so the result is the start of the
 * lowest hole of at least the rounded size.  Returns ORACLE_EINVAL for
 * request == 0 (or one that rounds past 2^64), else ORACLE_OK with
 * *offset_out = that start, or UINT64_MAX if no hole holds it. */
int oracle_first_fit(const uint64_t *offset, const uint64_t *size,
                     const uint8_t *live, uint64_t n, uint64_t arena_bytes,
                     uint64_t request, uint64_t *offset_out);

/* Layout monitor.  [CANN] 5.3 MemoryMonitor: usage = used / total; above
 * the critical ratio the level is CRITICAL, else above the warning ratio
 * WARNING, else OK; the time to exhaustion is the remaining bytes over the
 * growth rate, infinite when the rate is not positive.  [910C] monitoring
 * and the closing advice: when an allocation fails while enough is free,
 * look at the largest contiguous free block -- the layout, not the
 * capacity, is at fault; compaction is a costly stop-loss step.  Action:
 * with a pending request (rounded up to 32 bytes, [CANN] 2.2) that the
 * largest hole cannot hold, compact (targeted) if the free total could
 * hold it, else report that no compaction can help; otherwise compact
 * (full) when free/largest - 1 exceeds a threshold (> 0), else nothing. */
#define ORACLE_LEVEL_OK 0
#define ORACLE_LEVEL_WARNING 1
#define ORACLE_LEVEL_CRITICAL 2
#define ORACLE_ACTION_NONE 0
#define ORACLE_ACTION_TARGETED 1
#define ORACLE_ACTION_FULL 2
#define ORACLE_ACTION_NO_ROOM 3

typedef struct oracle_monitor_out {
    int32_t level;
    int32_t action;
    double usage_ratio;
    double frag_free_over_largest_minus_1;
    double seconds_to_full;
} oracle_monitor_out;

void oracle_monitor(uint64_t arena_bytes, uint64_t live_bytes, uint64_t largest_hole,
                    double warning_ratio, double critical_ratio, double frag_threshold,
                    uint64_t next_request, double growth_bytes_per_s,
                    oracle_monitor_out *out);

#ifdef __cplusplus
}
#endif

#endif

/*
 * arena_compaction.h -- in-place compaction of a device-memory arena on one
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the periodic compaction operator of the page "Ascend 910C
 * cluster tuning: memory-fragment compaction in mixed-precision training"
 * (section "Periodic compaction with Ascend C"): live tensors are known (the
 * caller marks them), holes are scanned from low to high addresses and every
 * live block gets its downward shift, the data moves, then every reference is
 * updated in one batch.  The free-space measures are that page's section
 * "Total-usage monitoring misses fragmentation" and section 3.2 of "CANN
 * memory management and memory optimisation" (fragmentation rate); the
 * post-state -- all allocated blocks contiguous, one large free region -- is
 * the periodic compaction of that page's section 3.3.
 *
 * Model
 *   arena   : caller-owned device bytes [0, S).
 *   table   : n entries (offset, size, live), structure of arrays in device
 *             memory, ascending by offset and non-overlapping.  Entries are
 *             32-byte aligned and non-empty (the CANN pool rounds every
 *             request up to 32 bytes, section 2.2; section 3.3 aligns to 32 or
 *             64 bytes).  Bytes not covered by a live entry -- free entries,
 *             untracked gaps, the tail -- are free; adjacent free bytes form
 *             one hole (the CANN pool merges adjacent free blocks, 2.2).
 *   result  : live blocks keep their order and are packed from offset 0:
 *             new_offset[i] = sum of sizes of live entries before i, for every
 *             entry (a free entry gets the value of the next live one).  With
 *             pinned entries (see defrag_table) the same holds inside every
 *             segment, from the segment's start, and a pinned entry keeps its
 *             offset.  A byte no moved block lands on is never written.
 *   handles : byte addresses in the arena.  A handle inside live block i maps
 *             to new_offset[i] + (h - offset[i]); any other handle (in a hole,
 *             at or past the arena end) maps to UINT64_MAX and is counted.
 *
 * Call order per compaction: defrag_plan (or defrag_plan_targeted) ->
 * defrag_move -> defrag_remap (any number of handle batches) ->
 * defrag_commit (optional: the packed table).  defrag_stats measures any
 * table without planning.
 *
 * Ownership: the caller owns every buffer (arena, table, outputs, handles and
 * the workspace).  The library allocates no device memory, creates no stream
 * or event, and never writes the table.  Its only process-wide state is a
 * counter for plan epochs, a per-device cache of the compute-unit count, and
 * a pool of small pinned host buffers (about 1 KiB each, one per call in
 * flight at a time, allocated on first need and kept until the process
 * ends) into which the calls that return figures read their results back;
 * defrag_compact_static uses none of them.
 *
 * Concurrency: between defrag_plan and the end of defrag_move nothing else
 * may read or write the arena, the table or the workspace (the 910C page runs
 * compaction while the affected tensors pause reads and writes -- a global
 * sync point).  defrag_remap and defrag_commit read the plan from the
 * workspace too, so until the last of them the workspace serves no other
 * call, except defrag_stats and defrag_first_fit (of any table): those
 * write only a statistics region of fixed size and a header of their own,
 * in front of the plan's data (defrag_compact's post-check is such a call).
 * Ordering is the stream's order;
 * calls on distinct workspaces are independent.  Every pointer argument
 * named "_dev" is device memory on the stream's device; "_host" is host
 * memory.
 *
 * Errors: negative return codes below.  Validation runs inside defrag_plan /
 * defrag_stats on the device before any output is written, so an invalid
 * table moves no byte and leaves new_offset untouched.
 */
#ifndef ARENA_COMPACTION_H
#define ARENA_COMPACTION_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DEFRAG_OK 0
#define DEFRAG_EINVAL (-1)     /* bad table or argument                        */
#define DEFRAG_EWORKSPACE (-2) /* workspace missing, misaligned or too small   */
#define DEFRAG_ENOPLAN (-3)    /* move/remap/commit without a matching plan     */
#define DEFRAG_EHIP (-4)       /* a HIP runtime call failed                    */
#define DEFRAG_ETIMEOUT (-5)   /* mover watchdog expired (a wait never ended)  */
#define DEFRAG_ENOFIT (-6)     /* no hole holds / no window frees the request  */
#define DEFRAG_ECAPACITY (-7)  /* a mover tile met more blocks than the launch
                                  gave it room for (the plan and the launch
                                  disagree; the arena is then undefined)       */
#define DEFRAG_ECORRUPT (-8)   /* the workspace no longer holds a consistent
                                  plan (overwritten since planning): tiles
                                  whose bytes or blocks fall outside the arena
                                  or the plan's arrays were not moved; the
                                  arena is then undefined                     */
#define DEFRAG_ETOOBIG (-9)    /* defrag_compact_static: the table needs more
                                  workspace than the library's static scratch
                                  (DEFRAG_STATIC_SCRATCH_BYTES) holds          */

/* Why a table was rejected: the first failing entry, and within it the first
 * failing check in the order zero size, misaligned, live flag, pinned flag,
 * out of arena, overlap. */
#define DEFRAG_REASON_NONE 0
#define DEFRAG_REASON_ZERO_SIZE 1     /* size == 0                              */
#define DEFRAG_REASON_MISALIGNED 2    /* offset or size not a multiple of 32    */
#define DEFRAG_REASON_LIVE_FLAG 3     /* live is neither 0 nor 1                */
#define DEFRAG_REASON_OUT_OF_ARENA 4  /* offset + size > arena bytes            */
#define DEFRAG_REASON_OVERLAP 5       /* starts before the previous entry ends  */
#define DEFRAG_REASON_ARGUMENT 6      /* a pointer or size argument (host side) */
#define DEFRAG_REASON_PINNED_FLAG 7   /* pinned not 0/1, or pinned but not live */

/* Largest supported table: entry indices are 32-bit inside the kernels. */
#define DEFRAG_MAX_ENTRIES 0xFFFFFFF0ull

typedef struct defrag_table {
    const uint64_t *offset_dev; /* n byte offsets from the arena base          */
    const uint64_t *size_dev;   /* n sizes in bytes                            */
    const uint8_t *live_dev;    /* n flags 0/1; NULL means every entry is live */
    uint64_t n;
    /* n flags 0/1; NULL means nothing is pinned.  A pinned entry must be
     * live; it never moves (910C page, "Cutting alloc and free at the
     * source": the parameter region keeps fixed addresses).  Pinned entries
     * split the arena into segments -- from one pinned block's end to the
     * next one's start, or to an arena end -- and each segment packs its
     * movable live blocks down to its own start. */
    const uint8_t *pinned_dev;
} defrag_table;

typedef struct defrag_stats_t {
    uint64_t arena_bytes;
    uint64_t live_bytes;   /* sum of live sizes                              */
    uint64_t free_bytes;   /* arena_bytes - live_bytes                       */
    uint64_t largest_hole; /* longest run of bytes outside live blocks       */
    uint64_t hole_count;   /* number of such runs                            */
    uint64_t live_blocks;
    uint64_t moved_blocks; /* live blocks whose new offset differs           */
    uint64_t moved_bytes;  /* their total size                               */
    /* free/largest - 1 (910C page, monitoring section); 0 when nothing free */
    double frag_free_over_largest_minus_1;
    /* 1 - largest/free (CANN page 3.2); 0 when nothing is free              */
    double frag_one_minus_largest_over_free;
    uint64_t invalid_index; /* first rejected entry, UINT64_MAX if valid     */
    int32_t invalid_reason; /* DEFRAG_REASON_*                               */
    int32_t reserved;
} defrag_stats_t;

/* Optional knobs.  Passing NULL takes the defaults: the tile size chosen by
 * the plan (below), streaming loads and stores, and one 512-lane mover
 * workgroup per compute unit (recorded in plan_host->tuning).  In a struct
 * passed explicitly, a zero tile size or spin limit takes its default and the
 * other fields are taken as given. */
typedef struct defrag_tuning {
    uint32_t tile_bytes;      /* mover tile: power of two in [256, 262144],
                                 or 0: the plan chooses on the device from the
                                 shifts it finds -- 131072 when more than half
                                 of the moved bytes shift by less than 8 MiB
                                 and at least 64 MiB move (a tile then often
                                 depends on one still being read; 128 KiB
                                 tiles are moved two per workgroup in flight,
                                 which hides that wait), or whenever the
                                 arena is at most 64 MiB (a step bound by
                                 latency, where half as many tiles wait less)
                                 or its entries average under 8 KiB of it
                                 (small blocks: each tile's block table then
                                 serves twice the bytes), else 65536 -- and
                                 the other one if the first's tiles do not
                                 fit the workspace.
                                 plan_host->tuning.tile_bytes says which.    */
    uint32_t wg_per_cu;       /* mover workgroups per compute unit; 0 means as
                                 many as the kernel's resources allow         */
    uint32_t nontemporal;     /* streaming hints: 0 none, 1 loads and stores,
                                 2 loads only, 3 stores only                 */
    uint32_t spin_limit_log2; /* mover watchdog: a wait gives up after
                                 2^x polls (default 22, a few seconds)       */
    /* Testing knob for the mover's dependency waits (0 = off); the result
     * does not change.  Tile t holds back its "sources read" flag -- the one
     * later tiles overwriting its sources wait for -- for stall_sleeps sleeps
     * of 127 x 64 clocks (about 3.4 us each at 2.4 GHz, at most 4096) when
     * h(t ^ stall_seed) % stall_every == 0, with h the 32-bit mix
     * x * 0x9E3779B1 then x ^ (x >> 15).  defrag_move_report counts the
     * waits that follow. */
    uint32_t stall_every;
    uint32_t stall_sleeps;
    uint32_t stall_seed;
    uint32_t reserved;        /* 0 */
} defrag_tuning;

/* Filled by defrag_plan (host memory, caller-owned).  Treat as opaque except
 * for .stats and the tuning fields wg_per_cu / nontemporal, which may be
 * changed before defrag_move. */
typedef struct defrag_plan_t {
    uint64_t magic;
    uint64_t epoch;
    const void *workspace;
    uint64_t workspace_bytes;
    uint64_t n;
    uint64_t arena_bytes;
    uint64_t live_blocks;
    uint64_t pinned_blocks;
    uint64_t move_begin;   /* lowest destination byte written by the move
                              (UINT64_MAX when nothing moves)                  */
    uint64_t live_bytes;
    uint64_t n_tiles;
    uint64_t max_tiles;    /* tile capacity of the workspace                   */
    uint64_t max_blocks_per_tile;
    uint64_t whole_tiles;  /* tiles that are one whole window of one block     */
    /* targeted plans (all 0 for a full plan): the request and the window
     * [window_begin, window_end) whose live blocks move; window_hole is the
     * hole it frees, at [window_end - window_hole, window_end) */
    uint64_t request_bytes;
    uint64_t window_begin;
    uint64_t window_end;
    uint64_t window_hole;
    int32_t state;         /* 0 none/invalid, 1 planned, 2 moved               */
    int32_t device;
    defrag_tuning tuning;
    defrag_stats_t stats;    /* of the table as planned (before the move)        */
} defrag_plan_t;

/* Workspace bytes for a table of n entries, at most max_pinned of them
 * pinned, over an arena of arena_bytes, with the given tile size (0: room
 * for the smaller size the plan may choose, 65536).  Returns 0 for impossible arguments, including an arena that
 * would need more than 0xFFFF0000 mover tiles (tile indices are 32-bit).  The workspace is device
 * memory, 256-byte aligned, owned by the caller; any content.  defrag_plan
 * uses whatever size it is given and returns DEFRAG_EWORKSPACE if the
 * table needs more mover tiles than fit. */
size_t defrag_workspace_bytes(uint64_t n, uint64_t max_pinned, uint64_t arena_bytes,
                              uint32_t tile_bytes);

/* Measure a table (910C monitoring: free total, largest contiguous free
 * block, both ratios; CANN 3.2).  Validates the table; on DEFRAG_EINVAL
 * out_host->invalid_index / invalid_reason say why.  Synchronises the
 * stream.  Ratios are IEEE binary64 computed on the host from the integers:
 * free/largest - 1 and 1 - largest/free, both 0 when free is 0. */
int defrag_stats(const defrag_table *table, uint64_t arena_bytes, void *ws_dev,
                 size_t ws_bytes, hipStream_t stream, defrag_stats_t *out_host);

/* First fit (CANN page, section 2.2 memory pool: a request is rounded up to
 * a multiple of 32 bytes and placed at the first free block that holds it;
 * adjacent free blocks are merged).  On a table the merged free blocks are
 * its holes in address order, so *offset_host receives the start of the
 * lowest hole of at least the rounded size.  This is the allocation the
 * 910C page's 4.2 GB buffer failed to get: ask before a compaction, and
 * again on the table defrag_commit writes after it.  Returns DEFRAG_OK, or
 * DEFRAG_ENOFIT with *offset_host = UINT64_MAX when no hole holds it;
 * DEFRAG_EINVAL for an invalid table (stats_host says why), a zero request
 * or one that rounds past 2^64.  stats_host (may be NULL) receives the
 * table's statistics, as defrag_stats.  The table is not changed: the
 * caller records the allocation.  Synchronises the stream. */
int defrag_first_fit(const defrag_table *table, uint64_t arena_bytes,
                     uint64_t request_bytes, void *ws_dev, size_t ws_bytes,
                     hipStream_t stream, uint64_t *offset_host,
                     defrag_stats_t *stats_host);

/* Plan a compaction (910C: scan holes low to high, give every live block its
 * downward shift).  Validates, writes new_offset_dev[n] (may be NULL), fills
 * *plan_host (including the stats of the table), and builds the mover's tile
 * table in the workspace.  Queues every pass, then synchronises once to
 * read a 256-byte header back.  tuning may be NULL. */
int defrag_plan(const defrag_table *table, uint64_t arena_bytes,
                const defrag_tuning *tuning, void *ws_dev, size_t ws_bytes,
                hipStream_t stream, uint64_t *new_offset_dev,
                defrag_plan_t *plan_host);

/* Plan a targeted compaction: move the fewest bytes that free one hole of at
 * least request_bytes (910C page, "Periodic compaction with Ascend C":
 * compaction pauses what it touches and is a stop-loss step; the failure it
 * answers is one request -- a 4.2 GB communication buffer -- that no free
 * block can hold).  A window is a run of consecutive holes with the live
 * blocks between them, none pinned; packing those blocks down to the
 * window's start merges its holes into one at its top.  The plan takes the
 * window whose hole holds the request with the fewest live bytes inside,
 * and among those the lowest; every live block outside it keeps its place,
 * so new_offset_dev is the segmented result with those blocks held (a
 * window already holding the request moves nothing).  Otherwise as
 * defrag_plan, and the plan feeds defrag_move / defrag_remap /
 * defrag_commit unchanged.  request_bytes == 0 is DEFRAG_EINVAL.  When no
 * window can free the request (it exceeds the largest hole a full
 * compaction would leave) returns DEFRAG_ENOFIT, writes nothing, and fills
 * plan_host->stats with the table's statistics, whose moved counts are
 * those of a full compaction.  Queues every pass, then synchronises once. */
int defrag_plan_targeted(const defrag_table *table, uint64_t arena_bytes,
                         uint64_t request_bytes, const defrag_tuning *tuning,
                         void *ws_dev, size_t ws_bytes, hipStream_t stream,
                         uint64_t *new_offset_dev, defrag_plan_t *plan_host);

/* Move the live blocks (910C: move the data).  arena_dev must be 16-byte
 * aligned and arena_bytes must equal the planned size.  Asynchronous; a plan
 * is consumed by one move (DEFRAG_ENOPLAN on reuse).  The table is not read:
 * everything comes from the plan's workspace. */
int defrag_move(void *arena_dev, uint64_t arena_bytes, defrag_plan_t *plan_host,
                void *ws_dev, size_t ws_bytes, hipStream_t stream);

/* After defrag_move: synchronise the stream and report whether the move
 * finished (DEFRAG_OK), or a wait timed out (DEFRAG_ETIMEOUT; the arena is
 * then undefined) or the workspace no longer held this plan
 * (DEFRAG_ENOPLAN; nothing moved), or held it damaged (DEFRAG_ECORRUPT) or
 * the launch had too little room for a tile's blocks (DEFRAG_ECAPACITY). */
int defrag_move_status(const defrag_plan_t *plan_host, const void *ws_dev,
                       hipStream_t stream);

/* After defrag_move (or defrag_compact): synchronise the stream and report
 * the move's outcome (status: what defrag_move_status returns) with the
 * mover's wait counters.  A tile is late when the flags of the earlier tiles
 * it must wait for were not all set when it first read them, right behind
 * its own loads; a late tile that then read one of them unset waited, and
 * polls counts those unset reads.  Returns DEFRAG_OK when the report is
 * filled (whatever the move's status), else an error as defrag_move_status.
 * Zeroed by the plan: valid until the workspace is planned again. */
typedef struct defrag_move_report_t {
    int32_t status;
    int32_t reserved;
    uint64_t tiles;
    uint64_t late_tiles;
    uint64_t waited_tiles;
    uint64_t polls;
} defrag_move_report_t;

int defrag_move_report(const defrag_plan_t *plan_host, const void *ws_dev,
                       hipStream_t stream, defrag_move_report_t *out_host);

/* Inspection of a plan's mover schedule, for tests and tools (the mover
 * itself needs no call).  The moved destination bytes are cut into tiles --
 * each the part of one run of consecutive moved blocks inside one
 * tile_bytes-aligned window -- in ascending order; a tile loads all its
 * sources, then stores once every earlier tile whose sources overlap its
 * destination has loaded (the plan's answer to the in-place hazards of the
 * 910C page's "Periodic compaction with Ascend C" move step).  Copies the
 * first min(cap, plan_host->n_tiles) tiles to out_host and synchronises the
 * stream.  Valid after defrag_plan and after defrag_move, until the
 * workspace is planned again (DEFRAG_ENOPLAN then). */
typedef struct defrag_tile_t {
    uint64_t dst_begin;    /* destination bytes [dst_begin, dst_end)          */
    uint64_t dst_end;
    uint64_t shift_first;  /* shift of the tile's first block                 */
    uint32_t first_block;  /* packed live-block indices (order of the table's */
    uint32_t last_block;   /* live entries) of the blocks the tile covers     */
    uint32_t dep_lo;       /* the earlier tiles it waits for, dep_lo..dep_hi; */
    uint32_t dep_hi;       /* none when dep_lo > dep_hi                       */
} defrag_tile_t;

int defrag_plan_tiles(const defrag_plan_t *plan_host, const void *ws_dev,
                      size_t ws_bytes, defrag_tile_t *out_host, uint64_t cap,
                      hipStream_t stream);

/* Remap handles (910C: update every reference in one batch).  h_out_dev may
 * equal h_in_dev.  *n_invalid_dev (may be NULL) receives the number of
 * handles mapped to UINT64_MAX.  Needs a valid plan of the table the handles
 * refer to (before or after the move).  Asynchronous.
 *
 * The remap is a function of the old table and its new offsets alone:
 * h inside live entry i maps to new_offset[i] + (h - offset[i]).  The plan
 * is where the library keeps that pair (the packed old offsets and shifts,
 * plus a bucket index over them), so the call takes the plan, not the
 * table: a caller holding only (old table, new_offset) plans that table
 * again (defrag_plan writes the same new_offset) and remaps through it.
 * The workspace must still hold the plan: remap every batch of handles
 * before the workspace is planned again. */
int defrag_remap(const defrag_plan_t *plan_host, const void *ws_dev,
                 size_t ws_bytes, const uint64_t *h_in_dev, uint64_t *h_out_dev,
                 uint64_t n_handles, uint64_t *n_invalid_dev, hipStream_t stream);

/* Write the packed table: the live_blocks entries (new offset, size, live
 * = 1, pinned flag) in order.  Any output pointer may be NULL.
 * Asynchronous. */
int defrag_commit(const defrag_plan_t *plan_host, const void *ws_dev,
                  size_t ws_bytes, uint64_t *offset_out_dev,
                  uint64_t *size_out_dev, uint8_t *live_out_dev,
                  uint8_t *pinned_out_dev, hipStream_t stream);

/* One whole compaction in one call -- the pages' operator: mark (the caller's
 * live flags), scan holes and plan, move, update every reference in one
 * batch (910C page, "Periodic compaction with Ascend C") -- then the
 * post-check (CANN page 3.3: one contiguous free region).  Runs
 * defrag_plan (or defrag_plan_targeted when request_bytes > 0),
 * defrag_move, defrag_remap (when n_handles or n_invalid_dev is given),
 * defrag_commit (when any packed-table output is given) and, when
 * after_host is given, defrag_stats of the packed table.  Everything runs
 * on `stream`.  The move is queued right behind the plan's passes, before
 * the plan is read back: it takes its tile count and workgroup count from
 * the plan in the workspace, and moves nothing if the plan failed.  Remap,
 * commit and the post-check, which read the plan and never the arena, run
 * in the first workgroups of the move's own launch, beside the movers (the
 * post-check with a header of its own in the workspace); one read at the
 * end brings the plan, the mover's status and the post-check.  With a NULL
 * or misaligned arena, a tuning of wg_per_cu 0, or
 * after_host without offset_out_dev and size_out_dev, the steps run in the
 * plain order instead (plan, read back, argument checks, move).  Returns
 * the first failing step's code (nothing moves if the plan fails;
 * DEFRAG_ETIMEOUT leaves the arena undefined).  plan_host is filled as by
 * the planning call and is consumed (state 2).  after_host needs
 * offset_out_dev and size_out_dev unless nothing is live (DEFRAG_EINVAL,
 * checked after the plan and before anything moves); pass pinned_out_dev
 * too so pinned blocks stay pinned in the post-check. */
typedef struct defrag_compact_args {
    const defrag_table *table;
    uint64_t arena_bytes;
    void *arena_dev;
    uint64_t request_bytes;        /* 0: full compaction; > 0: targeted       */
    const defrag_tuning *tuning;   /* may be NULL                             */
    void *ws_dev;
    size_t ws_bytes;
    uint64_t *new_offset_dev;      /* n entries, may be NULL                  */
    const uint64_t *h_in_dev;      /* handles (n_handles), may be NULL if 0   */
    uint64_t *h_out_dev;           /* may equal h_in_dev                      */
    uint64_t n_handles;
    uint64_t *n_invalid_dev;       /* may be NULL                             */
    uint64_t *offset_out_dev;      /* packed table, live_blocks entries each; */
    uint64_t *size_out_dev;        /* any may be NULL                         */
    uint8_t *live_out_dev;
    uint8_t *pinned_out_dev;
} defrag_compact_args;

int defrag_compact(const defrag_compact_args *args, hipStream_t stream,
                   defrag_plan_t *plan_host, defrag_stats_t *after_host);

/* defrag_compact for callers that cannot allocate device memory or create
 * streams and events: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is a device array the
 * library holds itself, DEFRAG_STATIC_SCRATCH_BYTES per GPU, from its load
 * to the end of the process; args->ws_dev and ws_bytes must be 0 (else
 * DEFRAG_EINVAL).  The steps run in defrag_compact's plain order on
 * `stream` alone (plan, read back, move, remap, commit, post-check, one
 * read at the end); the call calls no allocating routine and creates
 * nothing.  A table that needs more workspace than the scratch holds --
 * when defrag_workspace_bytes for it exceeds DEFRAG_STATIC_SCRATCH_BYTES,
 * it may -- returns DEFRAG_ETOOBIG before anything moves.  Every call on a
 * GPU uses that GPU's one array: calls that overlap on a GPU (from two
 * threads, or on two streams) race; serialise them.  The filled plan_host
 * describes the compaction but cannot be passed to calls that take a
 * workspace.  Otherwise as defrag_compact (same results, same errors). */
#define DEFRAG_STATIC_SCRATCH_BYTES (128ull << 20)

int defrag_compact_static(const defrag_compact_args *args, hipStream_t stream,
                          defrag_plan_t *plan_host, defrag_stats_t *after_host);

/* Layout monitor: host arithmetic on a defrag_stats result, no HIP call.
 * CANN page, section 5.3 (MemoryMonitor): usage = live / arena is rated OK,
 * WARNING above warning_ratio, CRITICAL above critical_ratio (defaults 0.85
 * and 0.95); seconds_to_full = free bytes / growth rate, +infinity for a
 * rate that is not positive.  910C page (monitoring section and closing
 * advice: read the largest free block next to the free total; compaction is
 * a stop-loss step): the action is
 *   TARGETED  a pending request, rounded up to 32 bytes as the CANN pool
 *             does (section 2.2), exceeds the largest hole but not the free
 *             total -- the layout is at fault (see defrag_plan_targeted,
 *             which may still find no window when pinned blocks split the
 *             free space);
 *   NO_ROOM   it exceeds the free total: compaction cannot help;
 *   FULL      otherwise, free/largest - 1 exceeds frag_threshold (> 0);
 *   NONE      otherwise.
 * Call it on a schedule (the 910C page scanned the layout every 100 steps).
 * cfg may be NULL (defaults, no request, no threshold).  Returns
 * DEFRAG_EINVAL for NULL stats/out, statistics of an invalid table or
 * inconsistent figures, or a NaN in cfg. */
#define DEFRAG_LEVEL_OK 0
#define DEFRAG_LEVEL_WARNING 1
#define DEFRAG_LEVEL_CRITICAL 2
#define DEFRAG_ACTION_NONE 0
#define DEFRAG_ACTION_TARGETED 1
#define DEFRAG_ACTION_FULL 2
#define DEFRAG_ACTION_NO_ROOM 3

typedef struct defrag_monitor_cfg {
    double warning_ratio;      /* usage above it: WARNING                     */
    double critical_ratio;     /* usage above it: CRITICAL                    */
    double frag_threshold;     /* free/largest - 1 above it: FULL; <= 0 off   */
    uint64_t next_request;     /* bytes the next allocation needs; 0: none    */
    double growth_bytes_per_s; /* live-byte growth rate                       */
} defrag_monitor_cfg;

typedef struct defrag_monitor_report {
    int32_t level;   /* DEFRAG_LEVEL_*  */
    int32_t action;  /* DEFRAG_ACTION_* */
    double usage_ratio;
    double frag_free_over_largest_minus_1;
    double frag_one_minus_largest_over_free;
    double seconds_to_full;
} defrag_monitor_report;

int defrag_monitor(const defrag_stats_t *stats, const defrag_monitor_cfg *cfg,
                   defrag_monitor_report *out);

/* Short text for a return code. */
const char *defrag_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ARENA_COMPACTION_H */

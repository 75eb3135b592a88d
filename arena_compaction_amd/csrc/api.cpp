// api.cpp -- the C-ABI entry points: argument checks, workspace layout,
// kernel launches and error mapping.  All arithmetic on the table and the
// arena runs in the kernels (plan.hip, move.hip, remap.hip); the host only
// turns two integers into the two fragmentation ratios (IEEE binary64).
#include <atomic>
#include <cstddef>
#include <cstring>
#include <mutex>

#include "../../include/arena_compaction.h"
#include "internal.h"

using namespace ac;

namespace {

constexpr uint64_t kPlanMagic = 0x4e414c5047415244ull;  // "DRAGPLAN"


std::atomic<uint64_t> g_epoch{0x9E3779B97F4A7C15ull};

int num_cus_of(int dev) {
    static std::mutex mu;
    static int cache[64] = {0};
    if (dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = v;
    }
    return cache[dev];
}

bool tile_ok(uint32_t t) { return t >= kMinTile && t <= kMaxTile && (t & (t - 1)) == 0; }

int check_table(const defrag_table *t) {
    if (!t) return DEFRAG_EINVAL;
    if (t->n > DEFRAG_MAX_ENTRIES) return DEFRAG_EINVAL;
    if (t->n && (!t->offset_dev || !t->size_dev)) return DEFRAG_EINVAL;
    return DEFRAG_OK;
}

int check_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return DEFRAG_EWORKSPACE;
    if (ws_bytes < need) return DEFRAG_EWORKSPACE;
    return DEFRAG_OK;
}

void arg_error(defrag_stats_t *o) {
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->invalid_index = kNone;
    o->invalid_reason = DEFRAG_REASON_ARGUMENT;
}

// Free total and largest hole -> the two ratios; 0 when nothing is free.
void fill_stats(defrag_stats_t *o, const WsHeader &h, uint64_t arena_bytes) {
    std::memset(o, 0, sizeof(*o));
    o->arena_bytes = arena_bytes;
    o->invalid_index = kNone;
    o->invalid_reason = DEFRAG_REASON_NONE;
    if (h.bad_key != kNone) {
        o->invalid_index = h.bad_key >> 3;
        o->invalid_reason = (int32_t)(h.bad_key & 7u);
        return;
    }
    o->live_bytes = h.live_bytes;
    o->free_bytes = arena_bytes - h.live_bytes;
    o->largest_hole = h.largest_hole;
    o->hole_count = h.hole_count;
    o->live_blocks = h.live_blocks;
    o->moved_blocks = h.moved_blocks;
    o->moved_bytes = h.moved_bytes;
    if (o->free_bytes == 0) {
        o->frag_free_over_largest_minus_1 = 0.0;
        o->frag_one_minus_largest_over_free = 0.0;
    } else {
        const double F = (double)o->free_bytes;
        const double L = (double)o->largest_hole;
        o->frag_free_over_largest_minus_1 = F / L - 1.0;
        o->frag_one_minus_largest_over_free = 1.0 - L / F;
    }
}

int read_header(WsHeader *out, const uint8_t *ws, const WsLayout &L, hipStream_t s) {
    return read_back(out, ws + L.header, sizeof(WsHeader), s);
}

TableView view_of(const defrag_table *t) {
    return TableView{t->offset_dev, t->size_dev, t->live_dev, t->pinned_dev, t->n};
}

WsLayout plan_layout(const defrag_plan_t *p) { return ws_with_tiles(p->n, p->max_tiles); }

int current_device() {
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess) return -1;
    return d;
}

// The mover's outcome from its status bits; 0 when it finished.
int move_outcome(const WsHeader &h, uint64_t epoch) {
    if (h.epoch != epoch) return DEFRAG_ENOPLAN;
    if (h.status & kStatusCorrupt) return DEFRAG_ECORRUPT;
    if (h.status & kStatusCapacity) return DEFRAG_ECAPACITY;
    if (h.status & kStatusTimeout) return DEFRAG_ETIMEOUT;
    return DEFRAG_OK;
}

int check_tuning(const defrag_tuning &tu) {
    if ((tu.tile_bytes && !tile_ok(tu.tile_bytes)) || tu.spin_limit_log2 > 40 || tu.nontemporal > 3 ||
        tu.stall_sleeps > kMaxStallSleeps)
        return DEFRAG_EINVAL;
    return DEFRAG_OK;
}

int check_plan(const defrag_plan_t *p, const void *ws, size_t ws_bytes) {
    if (!p || p->magic != kPlanMagic || p->state < 1) return DEFRAG_ENOPLAN;
    if (ws != p->workspace) return DEFRAG_ENOPLAN;
    if (ws_bytes < p->workspace_bytes) return DEFRAG_EWORKSPACE;
    if (current_device() != p->device) return DEFRAG_EINVAL;
    return DEFRAG_OK;
}

}  // namespace

extern "C" {

size_t defrag_workspace_bytes(uint64_t n, uint64_t max_pinned, uint64_t arena_bytes,
                              uint32_t tile_bytes) {
    const uint32_t T = tile_bytes ? tile_bytes : kDefaultTile;
    if (!tile_ok(T) || n > DEFRAG_MAX_ENTRIES || max_pinned > n) return 0;
    const uint64_t tiles = tiles_bound(arena_bytes, max_pinned, T);
    if (tiles > kMaxTiles) return 0;
    return ws_with_tiles(n, tiles).total;
}

}  // extern "C"

namespace {

// The statistics pass (and, if fit_need != kNone, the first fit).
int stats_pass(const defrag_table *table, uint64_t arena_bytes, uint64_t fit_need, void *ws_dev,
               size_t ws_bytes, hipStream_t stream, defrag_stats_t *out_host, WsHeader *h) {
    int rc = check_table(table);
    if (rc) {
        arg_error(out_host);
        return rc;
    }
    WsLayout L = ws_fixed(table->n);
    rc = check_ws(ws_dev, ws_bytes, L.tpart);  // the partial-result region only
    if (rc) {
        arg_error(out_host);
        return rc;
    }
    uint8_t *ws = static_cast<uint8_t *>(ws_dev);
    // the statistics header (the second 256 bytes): a plan the workspace
    // holds keeps its own header
    L.header = L.post;
    if (launch_stats_one(view_of(table), arena_bytes, ws, L, fit_need, false, stream) !=
        hipSuccess)
        return DEFRAG_EHIP;
    rc = read_header(h, ws, L, stream);
    if (rc) return rc;
    if (out_host) fill_stats(out_host, *h, arena_bytes);
    return h->bad_key == kNone ? DEFRAG_OK : DEFRAG_EINVAL;
}

// The post-check of the plain order (compact_serial), queued: the
// statistics pass of the packed table, with its own header (a plan's header
// is never written by it) and otherwise only the fixed statistics region in
// front of the plan's data; one launch, after the plan on this workspace.
int post_check_queue(const defrag_table *packed, uint64_t arena_bytes, void *ws_dev,
                     size_t ws_bytes, hipStream_t stream) {
    int rc = check_table(packed);
    if (rc) return rc;
    WsLayout L = ws_fixed(packed->n);
    rc = check_ws(ws_dev, ws_bytes, L.tpart);
    if (rc) return rc;
    uint8_t *ws = static_cast<uint8_t *>(ws_dev);
    L.header = L.post;
    return launch_stats_one(view_of(packed), arena_bytes, ws, L, kNone, true, stream) ==
                   hipSuccess
               ? DEFRAG_OK
               : DEFRAG_EHIP;
}

}  // namespace

extern "C" {

int defrag_stats(const defrag_table *table, uint64_t arena_bytes, void *ws_dev, size_t ws_bytes,
                 hipStream_t stream, defrag_stats_t *out_host) {
    if (!out_host) return DEFRAG_EINVAL;
    WsHeader h;
    return stats_pass(table, arena_bytes, kNone, ws_dev, ws_bytes, stream, out_host, &h);
}

int defrag_first_fit(const defrag_table *table, uint64_t arena_bytes, uint64_t request_bytes,
                     void *ws_dev, size_t ws_bytes, hipStream_t stream, uint64_t *offset_host,
                     defrag_stats_t *stats_host) {
    if (!offset_host) return DEFRAG_EINVAL;
    *offset_host = kNone;
    if (request_bytes == 0 || request_bytes > kNone - 31) {
        arg_error(stats_host);
        return DEFRAG_EINVAL;
    }
    const uint64_t need = (request_bytes + 31) / 32 * 32;
    WsHeader h;
    const int rc = stats_pass(table, arena_bytes, need, ws_dev, ws_bytes, stream, stats_host, &h);
    if (rc) return rc;
    *offset_host = h.fit_offset;
    return h.fit_offset == kNone ? DEFRAG_ENOFIT : DEFRAG_OK;
}

}  // extern "C"

namespace {

// A plan in flight: what its queued passes were given, for reading it back.
struct PlanCtx {
    WsLayout L;
    defrag_tuning tu;   // tile_bytes 0: chosen by the plan from `tiles`
    TileChoice tiles;
    bool tuned;  // the caller gave a tuning (else the plan picks workgroups)
    uint64_t epoch;
    int dev;
};

// Full plan (request == 0) or targeted plan (request > 0): check the
// arguments and queue every pass.  Nothing is read back.
// clear: a word the plan's last scan pass sets to zero, or null.
int plan_queue(const defrag_table *table, uint64_t arena_bytes, uint64_t request,
               const defrag_tuning *tuning, void *ws_dev, size_t ws_bytes, hipStream_t stream,
               uint64_t *new_offset_dev, defrag_plan_t *plan, PlanCtx *c,
               uint64_t *clear = nullptr) {
    if (!plan) return DEFRAG_EINVAL;
    std::memset(plan, 0, sizeof(*plan));
    defrag_tuning tu{};
    tu.wg_per_cu = kDefaultWgPerCu;
    tu.nontemporal = kDefaultNontemporal;
    if (tuning) tu = *tuning;
    if (!tu.spin_limit_log2) tu.spin_limit_log2 = kDefaultSpinLog2;
    if (check_tuning(tu)) {
        arg_error(&plan->stats);
        return DEFRAG_EINVAL;
    }
    int rc = check_table(table);
    if (rc) {
        arg_error(&plan->stats);
        return rc;
    }
    const uint64_t max_tiles = tiles_fitting(table->n, ws_bytes);
    rc = check_ws(ws_dev, ws_bytes, ws_fixed(table->n).fixed);
    if (rc || max_tiles == 0) {
        arg_error(&plan->stats);
        return DEFRAG_EWORKSPACE;
    }
    c->L = ws_with_tiles(table->n, max_tiles < kMaxTiles ? max_tiles : kMaxTiles);
    c->dev = current_device();
    if (c->dev < 0) return DEFRAG_EHIP;
    c->tu = tu;
    c->tiles = tu.tile_bytes ? TileChoice{tu.tile_bytes, tu.tile_bytes, 0u}
                             : TileChoice{kAutoTileSmall, kAutoTileLarge,
                                          auto_larger_always(arena_bytes, table->n) ? 1u : 0u};
    c->tuned = tuning != nullptr;
    uint8_t *ws = static_cast<uint8_t *>(ws_dev);
    c->epoch = g_epoch.fetch_add(0x9E3779B97F4A7C15ull) ^ reinterpret_cast<uintptr_t>(ws);
    const hipError_t e =
        request ? launch_targeted(view_of(table), arena_bytes, request, ws, c->L, new_offset_dev,
                                  c->tiles, c->epoch, clear, stream)
                : launch_scan(view_of(table), arena_bytes, ws, c->L, new_offset_dev, kOutNew,
                              c->tiles, c->epoch, kNone, clear, stream);
    return e == hipSuccess ? DEFRAG_OK : DEFRAG_EHIP;
}

// Fill the host plan from the header its passes wrote.
int plan_fill(const defrag_table *table, uint64_t arena_bytes, uint64_t request, void *ws_dev,
              const PlanCtx &c, const WsHeader &h, defrag_plan_t *plan) {
    fill_stats(&plan->stats, h, arena_bytes);
    if (h.bad_key != kNone) return DEFRAG_EINVAL;
    if (request && h.win_state != kWinFound) return DEFRAG_ENOFIT;  // nothing written
    if (h.n_tiles > c.L.max_tiles) return DEFRAG_EWORKSPACE;  // new offsets were written

    // the tile size the plan chose (one of the candidates)
    if (h.tile_bytes != c.tiles.a && h.tile_bytes != c.tiles.b) return DEFRAG_EHIP;
    defrag_tuning tu = c.tu;
    tu.tile_bytes = (uint32_t)h.tile_bytes;
    const uint64_t T = tu.tile_bytes;
    plan->epoch = c.epoch;
    plan->workspace = ws_dev;
    plan->workspace_bytes = c.L.total;
    plan->n = table->n;
    plan->arena_bytes = arena_bytes;
    plan->live_blocks = h.live_blocks;
    plan->pinned_blocks = h.pinned_blocks;
    plan->move_begin = h.move_begin;
    plan->live_bytes = h.live_bytes;
    plan->device = c.dev;
    plan->n_tiles = h.n_tiles;
    plan->max_tiles = c.L.max_tiles;
    // blocks meeting one tile: at most T / (smallest live size) + 2
    uint64_t mb = 1;
    if (h.min_live_size != kNone && h.min_live_size) mb = T / h.min_live_size + 2;
    if (mb > T / 32 + 2) mb = T / 32 + 2;
    plan->max_blocks_per_tile = mb;
    plan->whole_tiles = h.whole_tiles;
    plan->tuning = tu;
    if (request) {
        plan->request_bytes = request;
        plan->window_begin = h.win_begin;
        plan->window_end = h.win_end;
        plan->window_hole = h.win_hole;
    }
    plan->magic = kPlanMagic;
    plan->state = 1;
    return DEFRAG_OK;
}

int plan_common(const defrag_table *table, uint64_t arena_bytes, uint64_t request,
                const defrag_tuning *tuning, void *ws_dev, size_t ws_bytes, hipStream_t stream,
                uint64_t *new_offset_dev, defrag_plan_t *plan) {
    PlanCtx c;
    int rc = plan_queue(table, arena_bytes, request, tuning, ws_dev, ws_bytes, stream,
                        new_offset_dev, plan, &c);
    if (rc) return rc;
    WsHeader h;
    rc = read_header(&h, static_cast<uint8_t *>(ws_dev), c.L, stream);
    if (rc) return rc;
    return plan_fill(table, arena_bytes, request, ws_dev, c, h, plan);
}

// The end of a compaction: one read of the plan's header (the mover's
// status) and, after a post-check, of the statistics header beside it.
int compact_finish(const defrag_compact_args *a, hipStream_t stream, defrag_plan_t *plan,
                   defrag_stats_t *after_host, bool post_done) {
    const WsLayout L = plan_layout(plan);
    const uint8_t *ws = static_cast<const uint8_t *>(a->ws_dev);
    static_assert(sizeof(WsHeader) == 256, "two adjacent headers");
    WsHeader both[2];
    if (L.post != L.header + sizeof(WsHeader)) return DEFRAG_EHIP;
    const int rc = read_back(both, ws + L.header, (post_done ? 2 : 1) * sizeof(WsHeader), stream);
    if (rc) return rc;
    if (post_done) {
        fill_stats(after_host, both[1], a->arena_bytes);
        if (both[1].bad_key != kNone) return DEFRAG_EINVAL;
    }
    return plan->n_tiles ? move_outcome(both[0], plan->epoch) : DEFRAG_OK;
}

}  // namespace

namespace ac {

// The whole compaction in the plain order, every step on `stream` and
// nothing else created: plan (read back), the argument checks that need the
// plan, move, remap, commit, post-check, one read at the end.
int compact_serial(const defrag_compact_args *a, hipStream_t stream, defrag_plan_t *plan,
                   defrag_stats_t *after_host) {
    int rc = a->request_bytes
                 ? defrag_plan_targeted(a->table, a->arena_bytes, a->request_bytes, a->tuning,
                                        a->ws_dev, a->ws_bytes, stream, a->new_offset_dev, plan)
                 : defrag_plan(a->table, a->arena_bytes, a->tuning, a->ws_dev, a->ws_bytes,
                               stream, a->new_offset_dev, plan);
    if (rc) return rc;
    // the post-check reads the packed table (empty if nothing is live)
    if (after_host && plan->live_blocks && (!a->offset_out_dev || !a->size_out_dev)) {
        arg_error(after_host);
        return DEFRAG_EINVAL;  // checked before anything moves
    }
    rc = defrag_move(a->arena_dev, a->arena_bytes, plan, a->ws_dev, a->ws_bytes, stream);
    if (rc) return rc;
    if (a->n_handles || a->n_invalid_dev) {
        rc = defrag_remap(plan, a->ws_dev, a->ws_bytes, a->h_in_dev, a->h_out_dev, a->n_handles,
                          a->n_invalid_dev, stream);
        if (rc) return rc;
    }
    if (a->offset_out_dev || a->size_out_dev || a->live_out_dev || a->pinned_out_dev) {
        rc = defrag_commit(plan, a->ws_dev, a->ws_bytes, a->offset_out_dev, a->size_out_dev,
                           a->live_out_dev, a->pinned_out_dev, stream);
        if (rc) return rc;
    }
    if (after_host) {
        const defrag_table packed{a->offset_out_dev, a->size_out_dev, a->live_out_dev,
                                  plan->live_blocks, a->pinned_out_dev};
        rc = post_check_queue(&packed, a->arena_bytes, a->ws_dev, a->ws_bytes, stream);
        if (rc) {
            arg_error(after_host);
            return rc;
        }
    }
    return compact_finish(a, stream, plan, after_host, after_host != nullptr);
}

}  // namespace ac

extern "C" {

int defrag_plan(const defrag_table *table, uint64_t arena_bytes, const defrag_tuning *tuning,
                void *ws_dev, size_t ws_bytes, hipStream_t stream, uint64_t *new_offset_dev,
                defrag_plan_t *plan) {
    return plan_common(table, arena_bytes, 0, tuning, ws_dev, ws_bytes, stream, new_offset_dev,
                       plan);
}

int defrag_plan_targeted(const defrag_table *table, uint64_t arena_bytes, uint64_t request_bytes,
                         const defrag_tuning *tuning, void *ws_dev, size_t ws_bytes,
                         hipStream_t stream, uint64_t *new_offset_dev, defrag_plan_t *plan) {
    if (plan && request_bytes == 0) {
        std::memset(plan, 0, sizeof(*plan));
        arg_error(&plan->stats);
        return DEFRAG_EINVAL;
    }
    if (!plan) return DEFRAG_EINVAL;
    return plan_common(table, arena_bytes, request_bytes, tuning, ws_dev, ws_bytes, stream,
                       new_offset_dev, plan);
}

int defrag_move(void *arena_dev, uint64_t arena_bytes, defrag_plan_t *plan, void *ws_dev,
                size_t ws_bytes, hipStream_t stream) {
    int rc = check_plan(plan, ws_dev, ws_bytes);
    if (rc) return rc;
    if (plan->state != 1) return DEFRAG_ENOPLAN;
    if (arena_bytes != plan->arena_bytes) return DEFRAG_EINVAL;
    if (check_tuning(plan->tuning)) return DEFRAG_EINVAL;
    if (plan->n_tiles && (!arena_dev || (reinterpret_cast<uintptr_t>(arena_dev) & 15u)))
        return DEFRAG_EINVAL;
    plan->state = 2;
    if (plan->n_tiles == 0) return DEFRAG_OK;
    const int cus = num_cus_of(plan->device);
    if (cus <= 0) return DEFRAG_EHIP;
    const WsLayout L = plan_layout(plan);
    uint8_t *ws = static_cast<uint8_t *>(ws_dev);
    MoveArgs a{};
    a.arena = static_cast<uint8_t *>(arena_dev);
    a.live_dst = reinterpret_cast<const uint64_t *>(ws + L.live_dst);
    a.live_src = reinterpret_cast<const uint64_t *>(ws + L.live_src);
    a.tiles = reinterpret_cast<const TileRec *>(ws + L.tiles);
    a.flags = reinterpret_cast<uint32_t *>(ws + L.flags);
    a.hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    a.n_tiles = plan->n_tiles;
    a.epoch = plan->epoch;
    a.spin_limit = 1ull << plan->tuning.spin_limit_log2;
    a.tile_bytes = plan->tuning.tile_bytes;
    a.max_blocks = (uint32_t)plan->max_blocks_per_tile;
    a.small_blocks = move_small_blocks(plan->arena_bytes, plan->n) ? 1u : 0u;
    a.arena_bytes = arena_bytes;
    a.live_blocks = plan->live_blocks;
    a.stall_every = plan->tuning.stall_every;
    a.stall_sleeps = plan->tuning.stall_sleeps;
    a.stall_seed = plan->tuning.stall_seed;
    if (launch_move(a, plan->tuning.wg_per_cu, plan->tuning.nontemporal, cus, stream) !=
        hipSuccess)
        return DEFRAG_EHIP;
    return DEFRAG_OK;
}

int defrag_move_status(const defrag_plan_t *plan, const void *ws_dev, hipStream_t stream) {
    int rc = check_plan(plan, ws_dev, plan ? plan->workspace_bytes : 0);
    if (rc) return rc;
    if (plan->state != 2) return DEFRAG_ENOPLAN;
    if (plan->n_tiles == 0) {
        return hipStreamSynchronize(stream) == hipSuccess ? DEFRAG_OK : DEFRAG_EHIP;
    }
    const WsLayout L = plan_layout(plan);
    WsHeader h;
    rc = read_header(&h, static_cast<const uint8_t *>(ws_dev), L, stream);
    if (rc) return rc;
    return move_outcome(h, plan->epoch);
}

int defrag_move_report(const defrag_plan_t *plan, const void *ws_dev, hipStream_t stream,
                       defrag_move_report_t *out_host) {
    if (!out_host) return DEFRAG_EINVAL;
    std::memset(out_host, 0, sizeof(*out_host));
    int rc = check_plan(plan, ws_dev, plan ? plan->workspace_bytes : 0);
    if (rc) return rc;
    if (plan->state != 2) return DEFRAG_ENOPLAN;
    out_host->tiles = plan->n_tiles;
    if (plan->n_tiles == 0) {
        return hipStreamSynchronize(stream) == hipSuccess ? DEFRAG_OK : DEFRAG_EHIP;
    }
    WsHeader h;
    rc = read_header(&h, static_cast<const uint8_t *>(ws_dev), plan_layout(plan), stream);
    if (rc) return rc;
    out_host->status = move_outcome(h, plan->epoch);
    if (out_host->status == DEFRAG_ENOPLAN) return DEFRAG_ENOPLAN;
    out_host->late_tiles = h.late_tiles;
    out_host->waited_tiles = h.waited_tiles;
    out_host->polls = h.polls;
    return DEFRAG_OK;
}

int defrag_plan_tiles(const defrag_plan_t *plan, const void *ws_dev, size_t ws_bytes,
                      defrag_tile_t *out_host, uint64_t cap, hipStream_t stream) {
    int rc = check_plan(plan, ws_dev, ws_bytes);
    if (rc) return rc;
    const uint64_t k = cap < plan->n_tiles ? cap : plan->n_tiles;
    if (k && !out_host) return DEFRAG_EINVAL;
    const WsLayout L = plan_layout(plan);
    const uint8_t *ws = static_cast<const uint8_t *>(ws_dev);
    WsHeader h;
    rc = read_header(&h, ws, L, stream);
    if (rc) return rc;
    if (h.epoch != plan->epoch) return DEFRAG_ENOPLAN;  // planned again since
    if (k == 0) return DEFRAG_OK;
    // the device records are the public ones plus 8 bytes of padding
    static_assert(sizeof(defrag_tile_t) == 40 && sizeof(TileRec) == 48 &&
                      offsetof(TileRec, t0) == offsetof(defrag_tile_t, dst_begin) &&
                      offsetof(TileRec, t1) == offsetof(defrag_tile_t, dst_end) &&
                      offsetof(TileRec, shift0) == offsetof(defrag_tile_t, shift_first) &&
                      offsetof(TileRec, first_block) == offsetof(defrag_tile_t, first_block) &&
                      offsetof(TileRec, last_block) == offsetof(defrag_tile_t, last_block) &&
                      offsetof(TileRec, dep_lo) == offsetof(defrag_tile_t, dep_lo) &&
                      offsetof(TileRec, dep_hi) == offsetof(defrag_tile_t, dep_hi),
                  "tile record layouts");
    if (hipMemcpy2DAsync(out_host, sizeof(defrag_tile_t), ws + L.tiles, sizeof(TileRec),
                         sizeof(defrag_tile_t), k, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return DEFRAG_EHIP;
    return hipStreamSynchronize(stream) == hipSuccess ? DEFRAG_OK : DEFRAG_EHIP;
}

int defrag_remap(const defrag_plan_t *plan, const void *ws_dev, size_t ws_bytes,
                 const uint64_t *h_in_dev, uint64_t *h_out_dev, uint64_t n_handles,
                 uint64_t *n_invalid_dev, hipStream_t stream) {
    int rc = check_plan(plan, ws_dev, ws_bytes);
    if (rc) return rc;
    if (n_handles && (!h_in_dev || !h_out_dev)) return DEFRAG_EINVAL;
    const int cus = num_cus_of(plan->device);
    if (cus <= 0) return DEFRAG_EHIP;
    const WsLayout L = plan_layout(plan);
    const uint8_t *ws = static_cast<const uint8_t *>(ws_dev);
    if (launch_remap(ws, L, plan->arena_bytes, plan->n, plan->live_blocks, h_in_dev, h_out_dev,
                     n_handles, n_invalid_dev, cus, stream) != hipSuccess)
        return DEFRAG_EHIP;
    return DEFRAG_OK;
}

int defrag_commit(const defrag_plan_t *plan, const void *ws_dev, size_t ws_bytes,
                  uint64_t *offset_out_dev, uint64_t *size_out_dev, uint8_t *live_out_dev,
                  uint8_t *pinned_out_dev, hipStream_t stream) {
    int rc = check_plan(plan, ws_dev, ws_bytes);
    if (rc) return rc;
    const WsLayout L = plan_layout(plan);
    if (launch_commit(static_cast<const uint8_t *>(ws_dev), L, plan->live_blocks, offset_out_dev,
                      size_out_dev, live_out_dev, pinned_out_dev, stream) != hipSuccess)
        return DEFRAG_EHIP;
    return DEFRAG_OK;
}

int defrag_compact(const defrag_compact_args *a, hipStream_t stream, defrag_plan_t *plan,
                   defrag_stats_t *after_host) {
    if (!plan) return DEFRAG_EINVAL;
    if (!a || (a->n_handles && (!a->h_in_dev || !a->h_out_dev))) {
        std::memset(plan, 0, sizeof(*plan));
        arg_error(&plan->stats);
        return DEFRAG_EINVAL;
    }
    // Everything is queued at once on `stream` and sized on the device: the
    // move right behind the plan's passes, reading the tile count from the
    // plan's header; remap, commit and the post-check in the first
    // workgroups of the mover's launch, taking the live count from the same
    // header (a failed plan moves and writes nothing).  They read the plan,
    // never the arena, so they run while the move does.  One read of both
    // headers at the end fills the host plan.  That needs the arena and the
    // post-check's outputs known good before anything is queued, and a
    // workgroup count the device can pick; otherwise the calls run in the
    // plain order (plan, read back, check, move), which rejects a bad
    // argument before any byte moves.
    const bool arena_ok = a->arena_dev && !(reinterpret_cast<uintptr_t>(a->arena_dev) & 15u);
    const bool post_ok = !after_host || (a->offset_out_dev && a->size_out_dev);
    const bool wg_ok = !a->tuning || a->tuning->wg_per_cu != 0;
    if (!(arena_ok && post_ok && wg_ok)) return compact_serial(a, stream, plan, after_host);
    // the plan clears the invalid-handle count: the side job then only adds
    // to it
    PlanCtx c;
    int rc = plan_queue(a->table, a->arena_bytes, a->request_bytes, a->tuning, a->ws_dev,
                        a->ws_bytes, stream, a->new_offset_dev, plan, &c, a->n_invalid_dev);
    if (rc) return rc;
    const int cus = num_cus_of(c.dev);
    if (cus <= 0) return DEFRAG_EHIP;
    uint8_t *ws = static_cast<uint8_t *>(a->ws_dev);
    const WsHeader *gate = reinterpret_cast<const WsHeader *>(ws + c.L.header);
    const uint64_t n = a->table->n;  // the bound of every live count below
    MoveArgs m{};
    m.arena = static_cast<uint8_t *>(a->arena_dev);
    m.live_dst = reinterpret_cast<const uint64_t *>(ws + c.L.live_dst);
    m.live_src = reinterpret_cast<const uint64_t *>(ws + c.L.live_src);
    m.tiles = reinterpret_cast<const TileRec *>(ws + c.L.tiles);
    m.flags = reinterpret_cast<uint32_t *>(ws + c.L.flags);
    m.hdr = reinterpret_cast<WsHeader *>(ws + c.L.header);
    m.epoch = c.epoch;
    m.spin_limit = 1ull << c.tu.spin_limit_log2;
    m.tile_bytes = c.tiles.a;
    m.max_blocks = c.tiles.a / 32 + 2;  // the most blocks a tile can meet
    m.small_blocks = move_small_blocks(a->arena_bytes, n) ? 1u : 0u;
    m.device_sized = 1;
    m.wg_per_cu = c.tuned ? c.tu.wg_per_cu : 0;
    m.num_cus = (uint32_t)cus;
    m.max_tiles = c.L.max_tiles;
    m.arena_bytes = a->arena_bytes;
    m.live_blocks = n;  // room of the packed arrays; the count comes from the header
    m.stall_every = c.tu.stall_every;
    m.stall_sleeps = c.tu.stall_sleeps;
    m.stall_seed = c.tu.stall_seed;
    // with the tile size left to the plan, a mover for each candidate: the
    // one whose size the plan did not choose leaves at once -- unless the
    // plan takes the larger whatever the shifts (auto_larger_always; it
    // cuts fewer tiles, so it fits wherever the smaller would): then one
    // mover, of that size.
    MoveArgs mb = m;
    mb.tile_bytes = c.tiles.b;
    mb.max_blocks = c.tiles.b / 32 + 2;
    const bool one_mover = c.tiles.a == c.tiles.b || c.tiles.always_b;
    // Remap, commit and the post-check read the plan, never the arena: the
    // first workgroups of each mover's launch run them beside the move, in
    // the launch whose tile size the plan chose (the post-check takes the
    // packed table from the plan's packed arrays, the values the commit
    // writes).
    const bool want_commit =
        a->offset_out_dev || a->size_out_dev || a->live_out_dev || a->pinned_out_dev;
    const bool side_work = a->n_handles || a->n_invalid_dev || want_commit || after_host;
    const CommitOut out{a->offset_out_dev, a->size_out_dev, a->live_out_dev, a->pinned_out_dev};
    SideArgs sj = side_args(ws, c.L, a->arena_bytes, n, n, a->h_in_dev, a->h_out_dev,
                            a->n_handles, a->n_invalid_dev, want_commit ? &out : nullptr,
                            after_host != nullptr, gate, c.L.max_tiles);
    sj.any_tile = one_mover ? 1u : 0u;  // the one launch runs it
    const SideArgs *side = side_work ? &sj : nullptr;
    const MoveArgs &only = c.tiles.always_b ? mb : m;
    const bool ok =
        one_mover ? launch_move_device_sized(only, c.tu.nontemporal, side, stream) == hipSuccess
                  : launch_move_device_sized(m, c.tu.nontemporal, side, stream) == hipSuccess &&
                        launch_move_device_sized(mb, c.tu.nontemporal, side, stream) == hipSuccess;
    if (!ok) {
        // no kernel of this call still writes the caller's buffers once it returns
        (void)hipStreamSynchronize(stream);
        if (after_host) arg_error(after_host);
        return DEFRAG_EHIP;
    }
    // the plan's header (and the mover's status in it) and the post-check's
    static_assert(sizeof(WsHeader) == 256, "two adjacent headers");
    WsHeader both[2];
    if (c.L.post != c.L.header + sizeof(WsHeader)) return DEFRAG_EHIP;
    rc = read_back(both, ws + c.L.header, sizeof(both), stream);
    if (rc) return rc;
    rc = plan_fill(a->table, a->arena_bytes, a->request_bytes, a->ws_dev, c, both[0], plan);
    if (rc) return rc;
    plan->state = 2;
    if (after_host) {
        fill_stats(after_host, both[1], a->arena_bytes);
        if (both[1].bad_key != kNone) return DEFRAG_EINVAL;
    }
    return plan->n_tiles ? move_outcome(both[0], plan->epoch) : DEFRAG_OK;
}

const char *defrag_strerror(int code) {
    switch (code) {
        case DEFRAG_OK: return "ok";
        case DEFRAG_EINVAL: return "invalid table or argument";
        case DEFRAG_EWORKSPACE: return "workspace missing, misaligned or too small";
        case DEFRAG_ENOPLAN: return "no matching plan for this workspace";
        case DEFRAG_EHIP: return "HIP runtime error";
        case DEFRAG_ETIMEOUT: return "mover wait timed out";
        case DEFRAG_ENOFIT: return "no hole holds the request (and, for a targeted plan, no window can free it)";
        case DEFRAG_ECAPACITY: return "a mover tile met more blocks than its launch holds";
        case DEFRAG_ETOOBIG: return "the table needs more workspace than the library's static scratch holds";
        case DEFRAG_ECORRUPT: return "the workspace no longer holds a consistent plan (tiles outside it were not moved)";
        default: return "unknown error";
    }
}

}  // extern "C"

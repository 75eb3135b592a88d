// static.hip -- defrag_compact_static: the whole compaction for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Its workspace is a device array of the
// library's own, `scratch`, of fixed size; each GPU the library runs on holds
// one copy of it from the library's load to the end of the process.
//
// The steps are those of defrag_compact in its plain order (plan, read back,
// move, remap, commit, post-check, one read at the end), all on the caller's
// stream: the call creates no stream and no event and calls no allocating
// routine.  Every call on a GPU shares that GPU's array; the plan's own
// passes set every field and flag a later pass reads (its header fields,
// the mover's ticket, status and counters, each tile's flag), so nothing
// left by an earlier call is taken as input.  Calls that overlap on one GPU
// (two host threads, or two streams) race on the array.
#include <cstring>
#include <mutex>

#include "../../include/arena_compaction.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = DEFRAG_STATIC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address on the current device, looked up once per
// device with that device current: each GPU holds its own copy at its own
// address, and host code uses only that address (the array's name in host
// code is not a device address).
int scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DEFRAG_EHIP;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DEFRAG_EHIP;
        addr[dev] = p;
    }
    *out = addr[dev];
    return DEFRAG_OK;
}

void refuse(defrag_plan_t *plan) {
    std::memset(plan, 0, sizeof(*plan));
    plan->stats.invalid_index = ~0ull;
    plan->stats.invalid_reason = DEFRAG_REASON_ARGUMENT;
}

}  // namespace

extern "C" int defrag_compact_static(const defrag_compact_args *a, hipStream_t stream,
                                     defrag_plan_t *plan_host, defrag_stats_t *after_host) {
    if (!plan_host) return DEFRAG_EINVAL;
    // the scratch stands in for the workspace
    if (!a || a->ws_dev || a->ws_bytes ||
        (a->n_handles && (!a->h_in_dev || !a->h_out_dev))) {
        refuse(plan_host);
        return DEFRAG_EINVAL;
    }
    // a table whose plan arrays alone exceed the scratch: refused before
    // any HIP call (a plan that needs more tiles than fit beside them is
    // refused by the plan, on the device, before anything moves)
    if (a->table && a->table->n <= DEFRAG_MAX_ENTRIES &&
        ac::ws_fixed(a->table->n).fixed >= kScratchBytes) {
        refuse(plan_host);
        return DEFRAG_ETOOBIG;
    }
    void *ws = nullptr;
    const int rc0 = scratch_address(&ws);
    if (rc0) return rc0;
    defrag_compact_args b = *a;
    b.ws_dev = ws;
    b.ws_bytes = kScratchBytes;
    const ac::NoAllocScope no_alloc;  // its read-backs copy into pageable memory
    const int rc = ac::compact_serial(&b, stream, plan_host, after_host);
    return rc == DEFRAG_EWORKSPACE ? DEFRAG_ETOOBIG : rc;
}

// readback.cpp -- the read of a result header back to the host, the last
// step of every call that returns figures (plan, statistics, move status,
// the whole compaction).
//
// On a call of a few tens of microseconds the read-back is a large share:
// a copy into pageable host memory goes through a staging buffer and costs
// about 11 us beyond the stream's own wait, one into pinned memory about
// 3 us, and waiting in hipStreamSynchronize about 5 us more than watching a
// word in pinned memory.  So the headers are copied by a one-wave kernel
// into a pinned, device-mapped slot, followed by a sequence number stored
// with system-scope release; the host polls that word for a bounded time
// and then blocks in hipStreamSynchronize (which also reports a failed
// kernel) -- a long call, or one whose kernels failed, ends there.
//
// Slots come from a process-wide pool (one per call in flight, reused, never
// freed: pinned pages are few and small).  A thread inside a NoAllocScope
// (the entry point that allocates nothing) copies into its own pageable
// memory instead.
#include <atomic>
#include <chrono>
#include <cstddef>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/arena_compaction.h"
#include "internal.h"

namespace ac {
namespace {

constexpr uint32_t kSlotBytes = 1024;  // the most one read-back carries
constexpr auto kPollFor = std::chrono::microseconds(200);

struct HostSlot {
    uint64_t data[kSlotBytes / 8];
    uint64_t seq;        // written by the device: the last read-back completed
    uint64_t issued;     // host only: the last sequence number queued
    HostSlot *dev_addr;  // this slot as the device addresses it
};

std::mutex g_mu;
std::vector<HostSlot *> g_free;
thread_local int t_no_alloc = 0;

HostSlot *take_slot() {
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_free.empty()) {
            HostSlot *s = g_free.back();
            g_free.pop_back();
            return s;
        }
    }
    void *p = nullptr, *d = nullptr;
    if (hipHostMalloc(&p, sizeof(HostSlot),
                      hipHostMallocPortable | hipHostMallocMapped | hipHostMallocCoherent) !=
            hipSuccess ||
        !p)
        return nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || !d) {
        (void)hipHostFree(p);
        return nullptr;
    }
    std::memset(p, 0, sizeof(HostSlot));
    HostSlot *s = static_cast<HostSlot *>(p);
    s->dev_addr = static_cast<HostSlot *>(d);
    return s;
}

void give_slot(HostSlot *s) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_free.push_back(s);
}

int copy_pageable(void *out, const void *src, uint32_t bytes, hipStream_t s) {
    if (hipMemcpyAsync(out, src, bytes, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return DEFRAG_EHIP;
    return DEFRAG_OK;
}

}  // namespace

NoAllocScope::NoAllocScope() { ++t_no_alloc; }
NoAllocScope::~NoAllocScope() { --t_no_alloc; }

int read_back(void *out, const void *src_dev, uint32_t bytes, hipStream_t s) {
    if (bytes == 0 || bytes % 8 || bytes > kSlotBytes) return DEFRAG_EINVAL;
    if (t_no_alloc) return copy_pageable(out, src_dev, bytes, s);
    HostSlot *slot = take_slot();
    if (!slot) return copy_pageable(out, src_dev, bytes, s);
    const uint64_t seq = ++slot->issued;
    // the slot's fields at the device's address of it (address arithmetic only)
    char *dev = reinterpret_cast<char *>(slot->dev_addr);
    uint64_t *dev_data = reinterpret_cast<uint64_t *>(dev + offsetof(HostSlot, data));
    uint64_t *dev_seq = reinterpret_cast<uint64_t *>(dev + offsetof(HostSlot, seq));
    if (launch_publish(static_cast<const uint64_t *>(src_dev), dev_data, bytes / 8, dev_seq, seq,
                       s) != hipSuccess) {
        give_slot(slot);  // nothing was queued
        return DEFRAG_EHIP;
    }
    const auto t0 = std::chrono::steady_clock::now();
    bool seen = false;
    for (uint32_t k = 0;; ++k) {
        if (__atomic_load_n(&slot->seq, __ATOMIC_ACQUIRE) == seq) {
            seen = true;
            break;
        }
        if ((k & 255u) == 255u && std::chrono::steady_clock::now() - t0 > kPollFor) break;
    }
    if (!seen) {
        // a failed stream may still hold the copy: the slot leaves the pool
        if (hipStreamSynchronize(s) != hipSuccess) return DEFRAG_EHIP;
        if (__atomic_load_n(&slot->seq, __ATOMIC_ACQUIRE) != seq) return DEFRAG_EHIP;
    }
    std::memcpy(out, slot->data, bytes);
    give_slot(slot);
    return DEFRAG_OK;
}

}  // namespace ac

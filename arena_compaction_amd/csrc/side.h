// side.h -- the part of a compaction that reads the plan and never the
// arena: the handle remap, the packed table (commit) and the post-check
// (the statistics of the packed table), as one job for a range of
// workgroups.  It runs in a launch of its own (remap.hip: defrag_remap) or
// in the first workgroups of the one-call path's mover launch (move.hip),
// beside the move and with no second stream.
//
// Remap -- page "Ascend 910C cluster tuning: memory-fragment compaction in
// mixed-precision training", section "Periodic compaction with Ascend C"
// (after the data moves, every reference is updated in one batch) and
// section "Moving to other accelerators" (without a framework call that
// rewrites tensor addresses, references are kept at operator level).  A
// handle is a byte address in the arena and keeps its offset inside its
// block:
//   h inside live block j  ->  new_offset_j + (h - offset_j)
//   anything else          ->  UINT64_MAX (counted)
// One lane per handle, over the plan's packed live blocks (old offsets
// ascending), so free entries never cost a probe; a pinned block maps to
// itself.  Random handles make the search bound by L2 requests (each probe
// of each lane is its own cache line), so the plan builds an index -- the
// arena cut into at most 2^20 power-of-two buckets, each pointing at the
// first live block starting in it -- and each live block also has a search
// key (its old offset inside its bucket) and a record (old end, shift).  In
// arenas below 2^37 bytes with buckets of at most 2^32 bytes (the usual
// case) both fit in 32 bits and sit side by side in one 16-byte entry, so
// the probe that finds a block has its record too (kSideEnt); otherwise
// keys and records are separate arrays, the keys 32- or 64-bit and the
// records 8 or 16 bytes.  HBM traffic is 16 B per handle; the index and the
// entries stay in L2 / the last-level cache.
#ifndef ARENA_COMPACTION_SIDE_H
#define ARENA_COMPACTION_SIDE_H
#include "stats_one.h"

namespace ac {
namespace {

// One handle through the key-and-record entries: each probe that finds a
// block at or below h has read that block's record with its key, so the
// last such probe leaves the answer in registers; only a handle below the
// bucket's first block start reads a record afterwards, that of the block
// before the bucket.
__device__ inline uint64_t remap_one_ent(const SideArgs &s, uint64_t m, uint64_t h) {
    const RemapEnt *ent = static_cast<const RemapEnt *>(s.rec);
    const uint64_t b = h >> s.w;
    if (!m || b >= s.nb) return kNone;
    const uint64_t r0 = s.ridx[b];
    uint64_t first = r0, len = s.ridx[b + 1] - r0;
    const uint32_t hk = (uint32_t)(h & ((1ull << s.w) - 1));
    uint32_t end32 = 0, shift32 = 0;
    bool hit = false;
    while (len > 0) {
        const uint64_t half = len >> 1;
        const RemapEnt e = ent[first + half];
        if (e.key <= hk) {
            end32 = e.end32;
            shift32 = e.shift32;
            hit = true;
            first += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    if (!hit && r0 > 0) {  // the block before the bucket
        const RemapEnt e = ent[r0 - 1];
        end32 = e.end32;
        shift32 = e.shift32;
    }
    return h < ((uint64_t)end32 << 5) ? h - ((uint64_t)shift32 << 5) : kNone;
}

// One handle through separate keys and records.  The bucket of h gives the
// live blocks starting in it, [ridx[b], ridx[b+1]); the block holding h, if
// any, is the last one starting at or below h, found by a short search
// inside the bucket (or the block before it), and its record is one 8- or
// 16-byte read.  REC32: LiveRec32 records (arenas below 2^37 bytes).
template <bool REC32>
__device__ inline uint64_t remap_one(const SideArgs &s, uint64_t m, uint64_t h) {
    const uint64_t b = h >> s.w;
    if (!m || b >= s.nb) return kNone;
    uint64_t first = s.ridx[b], len = s.ridx[b + 1] - first;  // first with src > h
    if (s.key) {  // offsets inside the bucket, as 32-bit keys
        const uint32_t hk = (uint32_t)(h & ((1ull << s.w) - 1));
        while (len > 0) {
            const uint64_t half = len >> 1;
            if (s.key[first + half] <= hk) {
                first += half + 1;
                len -= half + 1;
            } else {
                len = half;
            }
        }
    } else {
        while (len > 0) {
            const uint64_t half = len >> 1;
            if (s.live_src[first + half] <= h) {
                first += half + 1;
                len -= half + 1;
            } else {
                len = half;
            }
        }
    }
    if (first == 0) return kNone;
    if constexpr (REC32) {  // the record of the last block starting at or below h
        const LiveRec32 r = static_cast<const LiveRec32 *>(s.rec)[first - 1];
        return h < ((uint64_t)r.end32 << 5) ? h - ((uint64_t)r.shift32 << 5) : kNone;
    } else {
        const LiveRec r = static_cast<const LiveRec *>(s.rec)[first - 1];
        return h < r.end ? h - r.shift : kNone;
    }
}

// Handles k0, k0 + stride, ...; returns how many mapped to nothing.
template <int KIND>
__device__ inline uint64_t remap_range(const SideArgs &s, uint64_t m, uint64_t k0,
                                       uint64_t stride) {
    uint64_t bad = 0;
    for (uint64_t k = k0; k < s.H; k += stride) {
        const uint64_t h = s.h_in[k];
        uint64_t out;
        if constexpr (KIND == kSideEnt) {
            out = remap_one_ent(s, m, h);
        } else {
            out = remap_one<KIND == kSideRec32>(s, m, h);
        }
        bad += (out == kNone) ? 1u : 0u;
        s.h_out[k] = out;
    }
    return bad;
}

// The job as run by workgroup g (of NT lanes) of s.groups.  Workgroup-
// uniform; the post-check's barriers inside.
template <int NT>
__device__ void side_part(const SideArgs &s, uint32_t g) {
    uint64_t m = s.m;
    if (s.gate) {  // queued before the plan was read back: its count, if it did not fail
        const uint64_t gm = s.gate->live_blocks;
        if (plan_failed(s.gate, s.max_tiles)) return;
        m = gm < m ? gm : m;
    }
    // the post-check first: its last workgroup to arrive has serial work
    // left, which the other workgroups' remap then overlaps
    if (s.post) {
        const TableView pt{s.lv.dst, s.lv.size, nullptr, s.lv.pin, m};  // all live
        // a step of NT lanes covers at most one scan tile of entries
        constexpr int kItems = NT >= (int)kScanTile ? 1 : (int)kScanTile / NT;
        stats_one_part<NT, kItems>(pt, m, s.arena_bytes, s.chunk, s.ngroups,
                                   static_cast<ChunkSum *>(s.csum), s.post_hdr, kNone, g);
    }
    const uint64_t stride = (uint64_t)s.groups * NT;
    const uint64_t k0 = (uint64_t)g * NT + threadIdx.x;
    if (s.commit) {  // packed entry k from the plan's packed arrays
        for (uint64_t k = k0; k < m; k += stride) {
            if (s.out.off) s.out.off[k] = s.lv.dst[k];
            if (s.out.size) s.out.size[k] = s.lv.size[k];
            if (s.out.live) s.out.live[k] = 1;
            if (s.out.pinned) s.out.pinned[k] = s.lv.pin[k];
        }
    }
    uint64_t bad = 0;
    if (s.kind == kSideEnt)
        bad = remap_range<kSideEnt>(s, m, k0, stride);
    else if (s.kind == kSideRec32)
        bad = remap_range<kSideRec32>(s, m, k0, stride);
    else
        bad = remap_range<kSideRec64>(s, m, k0, stride);
    if (s.n_invalid) {
        bad = wave_reduce(bad, add_op);
        if ((threadIdx.x & 63) == 0 && bad) atomicAdd(s.n_invalid, (unsigned long long)bad);
    }
}

}  // namespace
}  // namespace ac

#endif

// remap.hip -- handle remap for gfx950.
//
// Page: "Ascend 910C cluster tuning: memory-fragment compaction in
// mixed-precision training", section "Periodic compaction with Ascend C"
// (after the data moves, every reference is updated in one batch) and section
// "Moving to other accelerators" (without a framework call that rewrites
// tensor addresses, references are maintained at operator level).  A handle
// is a byte address in the arena; it keeps its offset inside its block:
//   h inside live block j  ->  new_offset_j + (h - offset_j)
//   anything else          ->  UINT64_MAX (counted)
//
// One lane per handle, grid-stride, over the plan's packed live blocks (old
// offsets ascending), so free entries never cost a probe; a pinned block
// maps to itself.  Random handles make the search bound by L2 requests (each
// probe of each lane is its own cache line), so the plan builds an index --
// the arena cut into at most 2^18 power-of-two buckets, each pointing at the
// first live block starting in it -- and each live block also has a search
// key (its old offset inside its bucket) and a record (old end, shift).  In
// arenas below 2^37 bytes with buckets of at most 2^32 bytes (the usual
// case) both fit in 32 bits and sit side by side in one 16-byte entry, so
// the probe that finds a block has its record too (k_remap_ent); otherwise
// keys and records are separate arrays, the keys 32- or 64-bit and the
// records 8 or 16 bytes (k_remap).  HBM traffic is 16 B per handle; the
// index and the entries stay in L2 / the last-level cache.
#include "stats_one.h"

namespace ac {
namespace {

constexpr uint32_t kRemapThreads = 256;
static_assert(kRemapThreads == kScanThreads, "the post-check runs as a scan workgroup");

// The one-call path's commit, done by the remap's launch: the packed live
// arrays and where the packed table goes.
struct CommitArgs {
    LiveView lv;
    CommitOut out;
};

// The post-check in the same launch: the statistics of the packed table,
// read from the plan's packed arrays (the values the commit writes).
struct PostArgs {
    uint64_t arena_bytes, chunk, ngroups;
    ChunkSum *cs;
    WsHeader *hdr;  // the statistics header
};

// Lanes k < m write packed entry k (grid-stride).
__device__ inline void commit_part(const CommitArgs &c, uint64_t m) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < m; k += stride) {
        if (c.out.off) c.out.off[k] = c.lv.dst[k];
        if (c.out.size) c.out.size[k] = c.lv.size[k];
        if (c.out.live) c.out.live[k] = 1;
        if (c.out.pinned) c.out.pinned[k] = c.lv.pin[k];
    }
}

__device__ inline void post_part(const CommitArgs &c, const PostArgs &post, uint64_t m) {
    const TableView pt{c.lv.dst, c.lv.size, nullptr, c.lv.pin, m, nullptr, 0};  // all live
    stats_one_part(pt, m, post.arena_bytes, post.chunk, post.ngroups, post.cs, post.hdr, kNone);
}

// One lane per handle, grid-stride.  The bucket of h gives the live blocks
// starting in it, [ridx[b], ridx[b+1]); the block holding h, if any, is the
// last one starting at or below h, so it is found by a short search inside
// the bucket (or is the block before it), and its record is one 8- or
// 16-byte read.  A random handle costs about three dependent cache-line requests:
// the index pair, a probe or two over the bucket's keys, the record.
// REC32: the records are LiveRec32 (arenas below 2^37 bytes), else LiveRec.
// COMMIT: the launch also writes the packed table (c); POST: and its
// statistics (workgroups below post.ngroups, before their handles).
template <bool REC32, bool COMMIT, bool POST>
__global__ __launch_bounds__(kRemapThreads) void k_remap(const void *__restrict__ rec,
                                                         const uint64_t *__restrict__ live_src,
                                                         const uint32_t *__restrict__ key,
                                                         const uint32_t *__restrict__ ridx,
                                                         uint32_t w, uint64_t nb, uint64_t m,
                                                         const uint64_t *h_in, uint64_t *h_out,
                                                         uint64_t H, unsigned long long *n_invalid,
                                                         const WsHeader *gate, uint64_t max_tiles,
                                                         CommitArgs c, PostArgs post) {
    if (gate) {  // queued before the plan was read back: its count, if it did not fail
        const uint64_t gm = gate->live_blocks;
        if (plan_failed(gate, max_tiles)) return;
        m = gm < m ? gm : m;
    }
    if constexpr (POST) post_part(c, post, m);
    if constexpr (COMMIT) commit_part(c, m);
    uint64_t bad = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < H; k += stride) {
        const uint64_t h = h_in[k];
        uint64_t out = kNone;
        const uint64_t b = h >> w;
        if (m && b < nb) {
            uint64_t first = ridx[b], len = ridx[b + 1] - first;  // first with src > h
            if (key) {  // offsets inside the bucket, as 32-bit keys
                const uint32_t hk = (uint32_t)(h & ((1ull << w) - 1));
                while (len > 0) {
                    const uint64_t half = len >> 1;
                    if (key[first + half] <= hk) {
                        first += half + 1;
                        len -= half + 1;
                    } else {
                        len = half;
                    }
                }
            } else {
                while (len > 0) {
                    const uint64_t half = len >> 1;
                    if (live_src[first + half] <= h) {
                        first += half + 1;
                        len -= half + 1;
                    } else {
                        len = half;
                    }
                }
            }
            if (first > 0) {  // the record of the last block starting at or below h
                if constexpr (REC32) {
                    const LiveRec32 r = static_cast<const LiveRec32 *>(rec)[first - 1];
                    if (h < ((uint64_t)r.end32 << 5)) out = h - ((uint64_t)r.shift32 << 5);
                } else {
                    const LiveRec r = static_cast<const LiveRec *>(rec)[first - 1];
                    if (h < r.end) out = h - r.shift;
                }
            }
        }
        bad += (out == kNone) ? 1u : 0u;
        h_out[k] = out;
    }
    if (n_invalid) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
        if ((threadIdx.x & 63) == 0 && bad) atomicAdd(n_invalid, (unsigned long long)bad);
    }
}

// The same with key and record side by side (RemapEnt): each probe that
// finds a block at or below h has read that block's record with its key, so
// the last such probe leaves the answer in registers; only a handle below
// the bucket's first block start reads a record afterwards, that of the
// block before the bucket.
template <bool COMMIT, bool POST>
__global__ __launch_bounds__(kRemapThreads) void k_remap_ent(const RemapEnt *__restrict__ ent,
                                                             const uint32_t *__restrict__ ridx,
                                                             uint32_t w, uint64_t nb, uint64_t m,
                                                             const uint64_t *h_in, uint64_t *h_out,
                                                             uint64_t H,
                                                             unsigned long long *n_invalid,
                                                             const WsHeader *gate,
                                                             uint64_t max_tiles, CommitArgs c,
                                                             PostArgs post) {
    if (gate) {  // queued before the plan was read back: its count, if it did not fail
        const uint64_t gm = gate->live_blocks;
        if (plan_failed(gate, max_tiles)) return;
        m = gm < m ? gm : m;
    }
    if constexpr (POST) post_part(c, post, m);
    if constexpr (COMMIT) commit_part(c, m);
    uint64_t bad = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < H; k += stride) {
        const uint64_t h = h_in[k];
        uint64_t out = kNone;
        const uint64_t b = h >> w;
        if (m && b < nb) {
            const uint64_t r0 = ridx[b];
            uint64_t first = r0, len = ridx[b + 1] - r0;
            const uint32_t hk = (uint32_t)(h & ((1ull << w) - 1));
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
            if (h < ((uint64_t)end32 << 5)) out = h - ((uint64_t)shift32 << 5);
        }
        bad += (out == kNone) ? 1u : 0u;
        h_out[k] = out;
    }
    if (n_invalid) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
        if ((threadIdx.x & 63) == 0 && bad) atomicAdd(n_invalid, (unsigned long long)bad);
    }
}

__global__ void k_zero_u64(uint64_t *p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

template <bool COMMIT, bool POST>
void remap_launch(const uint8_t *ws, const WsLayout &L, uint64_t arena_bytes, uint64_t n,
                  uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out, uint64_t n_handles,
                  unsigned long long *bad, const CommitArgs &c, const PostArgs &post,
                  const WsHeader *gate, uint64_t max_tiles, uint64_t grid, hipStream_t s) {
    const void *rec = ws + L.live_rec;
    const uint64_t *live_src = reinterpret_cast<const uint64_t *>(ws + L.live_src);
    const uint32_t *key = reinterpret_cast<const uint32_t *>(ws + L.live_key);
    const uint32_t *ridx = reinterpret_cast<const uint32_t *>(ws + L.ridx);
    const uint32_t *k32 = remap_keys32(arena_bytes, n) ? key : nullptr;
    const uint32_t w = remap_shift(arena_bytes, n);
    const uint64_t nb = remap_buckets(arena_bytes, n);
    if (remap_ent(arena_bytes, n))
        hipLaunchKernelGGL((k_remap_ent<COMMIT, POST>), dim3((uint32_t)grid), dim3(kRemapThreads),
                           0, s, static_cast<const RemapEnt *>(rec), ridx, w, nb, live_blocks,
                           h_in, h_out, n_handles, bad, gate, max_tiles, c, post);
    else if (remap_rec32(arena_bytes))
        hipLaunchKernelGGL((k_remap<true, COMMIT, POST>), dim3((uint32_t)grid),
                           dim3(kRemapThreads), 0, s, rec, live_src, k32, ridx, w, nb,
                           live_blocks, h_in, h_out, n_handles, bad, gate, max_tiles, c, post);
    else
        hipLaunchKernelGGL((k_remap<false, COMMIT, POST>), dim3((uint32_t)grid),
                           dim3(kRemapThreads), 0, s, rec, live_src, k32, ridx, w, nb,
                           live_blocks, h_in, h_out, n_handles, bad, gate, max_tiles, c, post);
}

}  // namespace

hipError_t launch_remap(const uint8_t *ws, const WsLayout &L, uint64_t arena_bytes, uint64_t n,
                        uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out,
                        uint64_t n_handles, uint64_t *n_invalid, const CommitOut *commit,
                        bool post, const WsHeader *gate, uint64_t max_tiles, int num_cus,
                        hipStream_t s) {
    if (n_invalid && !gate) {
        hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, s, n_invalid);
        AC_TRY(hipGetLastError());
    }
    const uint64_t work = (commit && live_blocks > n_handles) ? live_blocks : n_handles;
    PostArgs pa{arena_bytes, 0, 0, nullptr, nullptr};
    if (post) {  // the packed table has at most live_blocks entries
        const WsLayout F = ws_fixed(live_blocks);
        pa.chunk = F.scan_chunk;
        pa.ngroups = F.n_scan_blocks ? F.n_scan_blocks : 1;
        pa.cs = reinterpret_cast<ChunkSum *>(const_cast<uint8_t *>(ws) + L.csum);
        pa.hdr = reinterpret_cast<WsHeader *>(const_cast<uint8_t *>(ws) + L.post);
    }
    if (work == 0 && !post) return hipSuccess;
    uint64_t grid = (work + kRemapThreads - 1) / kRemapThreads;
    const uint64_t cap = (uint64_t)num_cus * 2;  // measured best of 1, 2, 3, 4, 8, 16 per CU
    if (grid > cap) grid = cap;
    if (grid < pa.ngroups) grid = pa.ngroups;
    unsigned long long *bad = reinterpret_cast<unsigned long long *>(n_invalid);
    CommitArgs c{live_view(ws, L), commit ? *commit : CommitOut{nullptr, nullptr, nullptr, nullptr}};
    if (commit && post)
        remap_launch<true, true>(ws, L, arena_bytes, n, live_blocks, h_in, h_out, n_handles, bad, c,
                                 pa, gate, max_tiles, grid, s);
    else if (commit)
        remap_launch<true, false>(ws, L, arena_bytes, n, live_blocks, h_in, h_out, n_handles, bad,
                                  c, pa, gate, max_tiles, grid, s);
    else if (post)
        remap_launch<false, true>(ws, L, arena_bytes, n, live_blocks, h_in, h_out, n_handles, bad,
                                  c, pa, gate, max_tiles, grid, s);
    else
        remap_launch<false, false>(ws, L, arena_bytes, n, live_blocks, h_in, h_out, n_handles, bad,
                                   c, pa, gate, max_tiles, grid, s);
    return hipGetLastError();
}

}  // namespace ac

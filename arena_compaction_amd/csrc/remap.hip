// remap.hip -- the side job's own launch (defrag_remap) and the host half
// of a side job: which search structures the plan built, and how many
// workgroups run it.  The job itself -- remap, commit, post-check -- is in
// side.h.
#include "side.h"

namespace ac {
namespace {

constexpr uint32_t kRemapThreads = 256;

__global__ __launch_bounds__(kRemapThreads) void k_side(SideArgs s) {
    side_part<kRemapThreads>(s, blockIdx.x);
}

__global__ void k_zero_u64(uint64_t *p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

}  // namespace

SideArgs side_args(const uint8_t *ws, const WsLayout &L, uint64_t arena_bytes, uint64_t n,
                   uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out,
                   uint64_t n_handles, uint64_t *n_invalid, const CommitOut *commit, bool post,
                   const WsHeader *gate, uint64_t max_tiles) {
    SideArgs s{};
    s.rec = ws + L.live_rec;
    s.live_src = reinterpret_cast<const uint64_t *>(ws + L.live_src);
    s.key = remap_keys32(arena_bytes, n) ? reinterpret_cast<const uint32_t *>(ws + L.live_key)
                                         : nullptr;
    s.ridx = reinterpret_cast<const uint32_t *>(ws + L.ridx);
    s.nb = remap_buckets(arena_bytes, n);
    s.w = remap_shift(arena_bytes, n);
    s.kind = remap_ent(arena_bytes, n) ? kSideEnt : remap_rec32(arena_bytes) ? kSideRec32
                                                                             : kSideRec64;
    s.h_in = h_in;
    s.h_out = h_out;
    s.H = n_handles;
    s.n_invalid = reinterpret_cast<unsigned long long *>(n_invalid);
    s.m = live_blocks;
    s.gate = gate;
    s.max_tiles = max_tiles;
    s.lv = live_view(ws, L);
    s.out = commit ? *commit : CommitOut{nullptr, nullptr, nullptr, nullptr};
    s.commit = commit ? 1u : 0u;
    s.post = post ? 1u : 0u;
    s.arena_bytes = arena_bytes;
    if (post) {
        s.csum = const_cast<uint8_t *>(ws) + L.csum;
        s.post_hdr = reinterpret_cast<WsHeader *>(const_cast<uint8_t *>(ws) + L.post);
    }
    s.work = (commit && live_blocks > n_handles) ? live_blocks : n_handles;
    return s;
}

void size_side(SideArgs &sj, uint32_t lanes, int num_cus) {
    uint64_t g = (sj.work + lanes - 1) / lanes;
    // measured best for the remap: 2 workgroups of 256 lanes per CU
    const uint64_t cap = ((uint64_t)num_cus * 512 + lanes - 1) / lanes;
    if (g > cap) g = cap;
    if (g > kMaxScanParts) g = kMaxScanParts;
    if (g < 1) g = 1;
    sj.groups = (uint32_t)g;
    if (sj.post) {
        // the packed table (at most m entries) in at most g chunks, each a
        // whole number of scan tiles (a step of the post-check's workgroup)
        const uint64_t tiles = (sj.m + kScanTile - 1) / kScanTile;
        const uint64_t per = tiles ? (tiles + g - 1) / g : 1;
        sj.chunk = per * kScanTile;
        sj.ngroups = tiles ? (tiles + per - 1) / per : 1;
    }
}

hipError_t launch_remap(const uint8_t *ws, const WsLayout &L, uint64_t arena_bytes, uint64_t n,
                        uint64_t live_blocks, const uint64_t *h_in, uint64_t *h_out,
                        uint64_t n_handles, uint64_t *n_invalid, int num_cus, hipStream_t s) {
    if (n_invalid) {
        hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, s, n_invalid);
        AC_TRY(hipGetLastError());
    }
    if (n_handles == 0) return hipSuccess;
    SideArgs sj = side_args(ws, L, arena_bytes, n, live_blocks, h_in, h_out, n_handles,
                            n_invalid, nullptr, false, nullptr, 0);
    size_side(sj, kRemapThreads, num_cus);
    hipLaunchKernelGGL(k_side, dim3(sj.groups), dim3(kRemapThreads), 0, s, sj);
    return hipGetLastError();
}

}  // namespace ac

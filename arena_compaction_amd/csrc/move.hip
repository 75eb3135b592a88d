// move.hip -- the in-place block mover for gfx950.
//
// Page: "Ascend 910C cluster tuning: memory-fragment compaction in
// mixed-precision training", section "Periodic compaction with Ascend C"
// (move the live data toward low addresses); "CANN memory management and
// memory optimisation", section 3.3 (periodic compaction gathers every
// allocated block into one contiguous region) and section 1.2 (data movement
// dominates and many small transfers cost far more than one large one -- so
// this is one fused kernel over all blocks, not a copy per block).
//
// Result: for every destination byte p below the live total, arena[p] takes
// the pre-move value of arena[p + shift(p)], where shift(p) is the downward
// shift of the live block landing on p.  Destination positions are packed,
// so the source position p + shift(p) rises strictly with p.
//
// Design.  The moved destinations form runs (one per segment between pinned
// blocks); each run is cut at every multiple of T into tiles, so a tile is
// at most one T-aligned window.  The plan records each tile's exact byte
// range, its blocks, and the earlier tiles it depends on.  Workgroups claim
// tiles in ascending order from an atomic ticket and, per tile:
//   1. load every 16-byte source vector of the tile into VGPRs (reads never
//      wait: a source byte can only be overwritten by the tile owning it as
//      a destination, which is at or above this tile and waits for it);
//   2. publish "sources read" for the tile;
//   3. wait until every earlier tile whose source range overlaps this tile's
//      destination has published (at most two tiles, found by the plan);
//   4. store.
// A wait only ever targets lower tickets, whose owners are running and whose
// reads never wait, so the schedule cannot deadlock and does not depend on
// how many workgroups are resident.  Self-overlap inside a tile is handled by
// the workgroup barrier between steps 1 and 4, so a move whose shift is far
// smaller than its size still runs in tile-sized waves spread over the whole
// chip rather than shift-sized serial steps.  Blocks whose shift is zero
// (pinned blocks, and the packed prefix of each segment) are in no tile and
// are never touched; nor is any byte no block lands on.
//
// Every tile, whole window of one block or not, takes one path with no
// branch around a memory access, so all of a lane's loads, and then all of
// its stores, stay in flight together (behind a per-vector branch the
// compiler waits for each store before the next): a lane outside the tile's
// range reloads the tile's first source vector, and stores go through a
// buffer descriptor over the tile's window, a disabled lane getting an
// offset the hardware drops as out of range.  (A separate straight-line
// path for whole single-block tiles, with global stores from uniform bases,
// was 0.8-1.0 points slower on the large workloads.)  The dependency flags
// are read once speculatively, right behind the tile's data loads: a
// dependency far below is long done, and the tile then stores without
// another round trip.
//
// Vectors are 16 bytes: offsets and sizes are multiples of 32, so a vector
// never straddles two blocks and both of its addresses are 16-byte aligned.
// Per tile the kernel reads 16 B per live-block descriptor it needs (in LDS
// only for tiles holding more than one block).
//
// The plan lives in caller memory.  When it has been read back to the host
// since it was written (defrag_move, a call of its own), a check pass runs
// first: every tile's bytes in one window inside the arena, its first source
// too, its blocks inside the packed arrays, its dependencies below it (else
// kStatusCorrupt), its blocks within the LDS the launch gives (else
// kStatusCapacity); on either the mover moves nothing.  A tile of several
// blocks also checks each vector's source against the arena (a lane that
// fails loads a safe vector instead and reports kStatusCorrupt).
// Queued right behind its own plan (defrag_compact) the mover takes the
// records as written.  The tile loop itself stays lean: each workgroup has
// one tile in flight, so every instruction between claiming a tile and
// issuing its loads, or between the loads' return and the stores, is paid
// on every tile (per-tile checks there cost 0.7% on the 80 GiB workload).
//
// Counters: a tile whose dependency flags were not all seen set behind its
// loads counts as late, and as waited if it then read a flag unset (with
// the number of such reads); all of it on the rare path.  A testing knob
// holds chosen tiles' flags back for a bounded time, so that later tiles do
// find them unset and the waits run at full size.
#include "side.h"

namespace ac {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Streaming hints: NT bit 0 marks loads, bit 1 marks stores non-temporal
// (the moved bytes are touched once; keeping them out of L2 leaves it to the
// tile table, descriptors and flags).
template <int NT>
__device__ __forceinline__ v4u load16(const uint8_t *p) {
    const v4u *q = reinterpret_cast<const v4u *>(p);
    if constexpr ((NT & 1) != 0) return __builtin_nontemporal_load(q);
    else return *q;
}

// Raw buffer resource (gfx9 family): word 3 of the descriptor, the
// non-temporal cache-policy bit of a buffer access, and an offset beyond any
// window (a buffer store out of range is dropped by the hardware).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kBufferNt = 2;
constexpr uint32_t kOutOfWindow = 0x80000000u;

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Wait-path testing knob: whether tile t holds its flag back (a 32-bit
// multiplicative mix of the tile index and a seed; 0 = off).
__device__ __forceinline__ bool stalls(uint32_t t, uint32_t every, uint32_t seed) {
    uint32_t h = (t ^ seed) * 0x9E3779B1u;
    h ^= h >> 15;
    return every != 0u && h % every == 0u;
}

// Before a move whose plan was read back to the host (and so could have been
// overwritten in the workspace since): every tile record checked against
// what a plan guarantees -- its bytes 16-byte aligned in one window inside
// the arena, its first block's sources (for a tile of one block, all of its
// sources) inside the arena, its blocks inside the packed arrays, its
// dependencies below it, its blocks within the LDS the launch gives -- one
// lane per tile.  A failure sets a status bit and the mover, queued behind,
// moves nothing.  (A tile of several blocks checks each vector's source
// itself: the block sizes it reads are not in its record.)
__global__ __launch_bounds__(256) void k_verify_tiles(MoveArgs a) {
    const uint64_t S = a.arena_bytes, T = a.tile_bytes, m = a.live_blocks;
    uint32_t bad = 0u, over = 0u;
    for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.n_tiles;
         t += (uint64_t)gridDim.x * blockDim.x) {
        const TileRec r = a.tiles[t];
        const uint64_t tb = r.t0 & ~(T - 1);
        const bool multi = r.first_block != r.last_block;
        const bool ok = ((r.t0 | r.t1 | r.shift0) & 15u) == 0 && r.t0 < r.t1 &&
                        r.t1 - tb <= T && r.shift0 < S && r.t1 <= S - r.shift0 &&
                        (r.dep_lo > r.dep_hi || r.dep_hi < t) &&
                        (!multi || (r.first_block < r.last_block && r.last_block < m));
        if (!ok) bad = 1u;
        else if (multi && r.last_block - r.first_block + 1u > a.max_blocks) over = 1u;
    }
    if (bad) atomicOr(&a.hdr->status, kStatusCorrupt);
    if (over) atomicOr(&a.hdr->status, kStatusCapacity);
}

// A tile as its record gives it to the workgroup: its window, the bytes of
// the window it writes, the earlier tiles it waits for, and whether its
// blocks fit the launch's LDS.
struct TileView {
    uint64_t tb;
    uint32_t rel0, rel1, dep_lo, dep_hi;
    bool ok;
};

// Mover workgroup wg's first ticket (0xFFFFFFFF when it takes part in
// nothing) into *s_ticket and the tile count into *s_ntiles; thread 0.
__device__ __forceinline__ void first_claim(const MoveArgs &a, uint32_t wg, uint32_t *s_ticket,
                                            uint64_t *s_ntiles) {
    // a workspace re-planned since this plan: move nothing, write nothing
    // (the status query sees the epoch mismatch); nor when the records
    // failed their check
    uint32_t tk = 0xFFFFFFFFu;
    const WsHeader *h = a.hdr;
    // every header field needed here is loaded before any is tested: one
    // memory round trip in front of the first claim, not one per field
    const uint64_t ep = __hip_atomic_load(&h->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t st = h->status;
    uint64_t nt = a.n_tiles, bad = kNone, win = kWinNone, tb = a.tile_bytes;
    if (a.device_sized) {
        nt = h->n_tiles;
        bad = h->bad_key;
        win = h->win_state;
        tb = h->tile_bytes;
    }
    bool go = (ep == a.epoch) & ((st & (kStatusCorrupt | kStatusCapacity)) == 0u);
    if (a.device_sized) {
        // the plan's results, read here instead of on the host: a failed
        // plan (invalid table, no window, too many tiles) moves nothing, nor
        // does the mover of a tile size the plan did not choose; workgroups
        // past the chosen count leave
        const uint32_t per_cu = a.wg_per_cu ? a.wg_per_cu : kDefaultWgPerCu;
        go = go & (bad == kNone) & (win != kWinNoFit) & (nt <= a.max_tiles) &
             (tb == a.tile_bytes) & (wg < (uint64_t)per_cu * a.num_cus);
    }
    if (go) tk = atomicAdd(&a.hdr->ticket, 1u);
    *s_ticket = tk;
    *s_ntiles = nt;
}

// Start tile t: read its record, stage the shifts and starts of a tile of
// several blocks in LDS, and issue every 16-byte source load into v (still
// in flight on return).
template <int THREADS, int VPT, int NT>
__device__ __forceinline__ TileView load_tile(const MoveArgs &a, uint32_t t, v4u (&v)[VPT],
                                              uint64_t *s_shift, uint32_t *s_rel) {
    const uint32_t tid = threadIdx.x;
    // The record is the same for every lane: make each field wave-uniform
    // (one wait for the record, scalar registers after) -- otherwise the
    // compiler waits for the record again before every data load below.
    const TileRec &rp = a.tiles[t];
    const uint64_t t0 = uniform64(rp.t0);
    const uint64_t t1 = uniform64(rp.t1);
    const uint64_t shift0 = uniform64(rp.shift0);
    const uint32_t first = __builtin_amdgcn_readfirstlane(rp.first_block);
    const uint32_t last = __builtin_amdgcn_readfirstlane(rp.last_block);
    TileView d;
    d.dep_lo = __builtin_amdgcn_readfirstlane(rp.dep_lo);
    d.dep_hi = __builtin_amdgcn_readfirstlane(rp.dep_hi);
    d.tb = t0 & ~((uint64_t)a.tile_bytes - 1);  // the tile's window
    d.rel0 = (uint32_t)(t0 - d.tb);
    d.rel1 = (uint32_t)(t1 - d.tb);
    const uint32_t nblk = last - first + 1u;
    d.ok = nblk <= a.max_blocks;  // LDS room (checked again; the plan sized it)

    if (nblk > 1u && d.ok) {
        for (uint32_t k = tid; k < nblk; k += THREADS) {
            const uint64_t dst = a.live_dst[first + k];
            s_shift[k] = a.live_src[first + k] - dst;
            s_rel[k] = dst <= d.tb ? 0u : (uint32_t)(dst - d.tb);
        }
        __syncthreads();
    }

    // no branch around a memory access: a lane outside [rel0, rel1) reloads
    // the tile's first source vector and discards it; so does a lane of a
    // tile of several blocks whose source would leave the arena (the blocks'
    // shifts come from the packed arrays, which the check pass does not
    // read) -- and reports it
    const uint8_t *first_src = a.arena + d.tb + d.rel0 + shift0;
    const uint64_t lim = a.arena_bytes - 16u - d.tb;  // largest source offset from tb
    bool lane_bad = false;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t r = ((uint32_t)j * THREADS + tid) * 16u;
        bool in = d.ok && r >= d.rel0 && r < d.rel1;
        uint64_t sh = shift0;
        if (nblk > 1u && d.ok) {
            uint32_t lo = 0, n = nblk;  // largest k with s_rel[k] <= r
            while (n > 1u) {
                const uint32_t half = n >> 1;
                lo = (s_rel[lo + half] <= r) ? lo + half : lo;
                n -= half;
            }
            sh = s_shift[lo];
            const bool inside = (sh & 15u) == 0 && sh <= lim && (uint64_t)r <= lim - sh;
            lane_bad |= in && !inside;
            in = in && inside;
        }
        v[j] = load16<NT>(in ? a.arena + d.tb + r + sh : first_src);
    }
    if (__builtin_expect(lane_bad, 0)) atomicOr(&a.hdr->status, kStatusCorrupt);
    return d;
}

// Thread 0, once every source load of tile t has returned: publish its
// "sources read" flag (the testing knob may hold it back first).
__device__ __forceinline__ void publish_tile(const MoveArgs &a, uint32_t t, bool ok) {
    if (!ok) atomicOr(&a.hdr->status, kStatusCapacity);
    if (__builtin_expect(a.stall_every != 0u, 0) && stalls(t, a.stall_every, a.stall_seed)) {
        for (uint32_t k = 0; k < a.stall_sleeps; ++k) __builtin_amdgcn_s_sleep(127);
    }
    __hip_atomic_store(&a.flags[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: wait until every tile in [dep_lo, dep_hi] has published (one
// seen set already -- f_lo for dep_lo, f_hi for dep_hi -- is not looked at
// again; look_first: take that first look here).  Returns 1 when the tile
// must not store: a wait gave up (status timeout) or its blocks do not fit
// the LDS.  A tile whose dependencies were not all seen done at the first
// look counts as late, and as waited if it polled.
__device__ __forceinline__ uint32_t wait_deps(const MoveArgs &a, uint32_t dep_lo, uint32_t dep_hi,
                                              uint32_t f_lo, uint32_t f_hi, bool ok,
                                              bool look_first) {
    if (look_first && dep_lo <= dep_hi) {
        f_lo = __hip_atomic_load(&a.flags[dep_lo], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f_hi = __hip_atomic_load(&a.flags[dep_hi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t skip = ok ? 0u : 1u;
    // the common case -- no dependency, or the one or two seen done behind
    // the data loads -- skips the polling loop, marked unlikely so the
    // compiler keeps the tile's path straight (measured: +0.6 points on the
    // 80 GiB workload, +1.0 on the self-overlapping one)
    const bool seen = dep_lo > dep_hi || (dep_hi - dep_lo <= 1u && f_lo && f_hi);
    if (__builtin_expect(!seen && !skip, 0)) {
        uint64_t polls = 0;
        for (uint32_t u = dep_lo; u <= dep_hi && !skip; ++u) {
            if ((u == dep_lo && f_lo) || (u == dep_hi && f_hi)) continue;  // seen done
            uint64_t p = 0;
            while (__hip_atomic_load(&a.flags[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
                if (++p > a.spin_limit) {
                    skip = 1u;
                    atomicOr(&a.hdr->status, kStatusTimeout);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            polls += p;
        }
        atomicAdd(reinterpret_cast<unsigned long long *>(&a.hdr->late_tiles), 1ull);
        if (polls) {
            atomicAdd(reinterpret_cast<unsigned long long *>(&a.hdr->waited_tiles), 1ull);
            atomicAdd(reinterpret_cast<unsigned long long *>(&a.hdr->polls),
                      (unsigned long long)polls);
        }
    }
    return skip;
}

// Buffer stores over the tile's window: a lane outside [rel0, rel1) gets an
// offset past the window's end, which the hardware drops -- no branch around
// any store.
template <int THREADS, int VPT, int NT>
__device__ __forceinline__ void store_tile(const MoveArgs &a, const TileView &d,
                                           const v4u (&v)[VPT]) {
    const __amdgpu_buffer_rsrc_t win =
        __builtin_amdgcn_make_buffer_rsrc(a.arena + d.tb, 0, (int)a.tile_bytes, kBufferRsrcWord3);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t r = ((uint32_t)j * THREADS + threadIdx.x) * 16u;
        const uint32_t off = (r >= d.rel0 && r < d.rel1) ? r : kOutOfWindow;
        __builtin_amdgcn_raw_buffer_store_b128(v[j], win, (int)off, 0, (NT & 2) ? kBufferNt : 0);
    }
}

// The tiles as moved by mover workgroup wg of a launch: one tile at a time.
template <int THREADS, int VPT, int NT>
__device__ __forceinline__ void move_tiles(const MoveArgs &a, uint32_t wg) {
    extern __shared__ uint64_t lds_dyn[];
    uint64_t *s_shift = lds_dyn;                                           // [max_blocks]
    uint32_t *s_rel = reinterpret_cast<uint32_t *>(lds_dyn + a.max_blocks);  // [max_blocks]
    __shared__ uint32_t s_ticket;
    __shared__ uint32_t s_skip;
    __shared__ uint64_t s_ntiles;
    const uint32_t tid = threadIdx.x;
    if (tid == 0) first_claim(a, wg, &s_ticket, &s_ntiles);
    __syncthreads();
    const uint64_t n_tiles = s_ntiles;
    uint32_t t = s_ticket;

    while (t < n_tiles) {
        v4u v[VPT];
        const TileView d = load_tile<THREADS, VPT, NT>(a, t, v, s_shift, s_rel);
        // first look at the dependency flags, returned with the data loads
        uint32_t f_lo = 0u, f_hi = 0u;
        if (tid == 0 && d.dep_lo <= d.dep_hi) {
            f_lo = __hip_atomic_load(&a.flags[d.dep_lo], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            f_hi = __hip_atomic_load(&a.flags[d.dep_hi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // every load of this tile has returned before its flag is published
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            publish_tile(a, t, d.ok);
            s_skip = wait_deps(a, d.dep_lo, d.dep_hi, f_lo, f_hi, d.ok, false);
        }
        __syncthreads();
        if (!s_skip) store_tile<THREADS, VPT, NT>(a, d, v);
        // Claim the next tile only now: each workgroup holds one ticket at a
        // time, which keeps the tiles in flight in one narrow window of the
        // arena (measured: about 2% more bandwidth than claiming early).
        if (tid == 0) s_ticket = atomicAdd(&a.hdr->ticket, 1u);
        __syncthreads();
        t = s_ticket;
    }
}

// The same with two tiles per workgroup in flight: the next tile (B) is
// claimed and its loads issued before the current one (A) waits for the
// tiles it depends on and stores, so by the time A looks at its
// dependencies they have nearly always published (a neighbour a short shift
// away published while B's loads ran).  Every wait still targets lower
// tickets only: A's dependencies lie below A < B, and the lowest ticket not
// yet published is some workgroup's B, whose A waits on published tickets
// alone, so the schedule cannot deadlock.  Used for 128 KiB tiles of
// 512 lanes, where two tiles fit one lane's registers: there it beats one
// tile at a time at every shift measured (short shifts 74 -> 83% of the HBM
// peak, long ones 82 -> 84%); with 64 KiB tiles the doubled window of
// tickets in flight costs more than it saves.
template <int THREADS, int VPT, int NT>
__device__ __forceinline__ void move_tiles_two(const MoveArgs &a, uint32_t wg) {
    extern __shared__ uint64_t lds_dyn[];
    uint64_t *s_shift = lds_dyn;                                           // [max_blocks]
    uint32_t *s_rel = reinterpret_cast<uint32_t *>(lds_dyn + a.max_blocks);  // [max_blocks]
    __shared__ uint32_t s_ticket;
    __shared__ uint32_t s_skip;
    __shared__ uint64_t s_ntiles;
    const uint32_t tid = threadIdx.x;
    if (tid == 0) first_claim(a, wg, &s_ticket, &s_ntiles);
    __syncthreads();
    const uint64_t n_tiles = s_ntiles;
    uint32_t tA = s_ticket;
    if (tA >= n_tiles) return;  // (the whole workgroup)
    v4u vA[VPT];
    TileView dA = load_tile<THREADS, VPT, NT>(a, tA, vA, s_shift, s_rel);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) publish_tile(a, tA, dA.ok);
    for (;;) {
        if (tid == 0) s_ticket = atomicAdd(&a.hdr->ticket, 1u);
        __syncthreads();
        const uint32_t tB = s_ticket;
        const bool haveB = tB < n_tiles;
        v4u vB[VPT];
        TileView dB{};
        // (the LDS table is A's no longer: its loads have returned)
        if (haveB) dB = load_tile<THREADS, VPT, NT>(a, tB, vB, s_shift, s_rel);
        if (tid == 0) s_skip = wait_deps(a, dA.dep_lo, dA.dep_hi, 0u, 0u, dA.ok, true);
        __syncthreads();
        if (!s_skip) store_tile<THREADS, VPT, NT>(a, dA, vA);
        if (!haveB) break;
        // every load of B has returned before its flag is published
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) publish_tile(a, tB, dB.ok);
        tA = tB;
        dA = dB;
#pragma unroll
        for (int j = 0; j < VPT; ++j) vA[j] = vB[j];
    }
}

// Which loop moves a launch's tiles (see move_tiles_two).
template <int THREADS, int VPT>
constexpr bool kTwoInFlight = THREADS == 512 && VPT == 16;

template <int THREADS, int VPT, int NT>
__device__ __forceinline__ void move_launch_tiles(const MoveArgs &a, uint32_t wg) {
    if constexpr (kTwoInFlight<THREADS, VPT>) move_tiles_two<THREADS, VPT, NT>(a, wg);
    else move_tiles<THREADS, VPT, NT>(a, wg);
}

template <int THREADS, int VPT, int NT>
__global__ __launch_bounds__(THREADS) void k_move(MoveArgs a) {
    move_launch_tiles<THREADS, VPT, NT>(a, blockIdx.x);
}

// The one-call path's mover: its first side.groups workgroups run the side
// job (remap, commit, post-check) instead, if the plan chose this mover's
// tile size (or side.any_tile), and the movers are the workgroups after
// them.  Registers are capped so that a side workgroup and a mover fit on
// one CU together (a SIMD's 512 VGPRs over two workgroups' waves: 128 a lane
// at 512 lanes, 64 at 1024), unless the mover's tile data alone would not
// fit in that (those run on CUs of their own).
template <int THREADS, int VPT>
constexpr int side_waves_per_eu() {
    constexpr int data = (kTwoInFlight<THREADS, VPT> ? 2 : 1) * VPT * 4;  // VGPRs of tile data
    return data + 32 < 65536 / THREADS ? THREADS / 128 : 1;
}
template <int THREADS, int VPT, int NT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(side_waves_per_eu<THREADS, VPT>()))) void k_move_side(
    MoveArgs a, SideArgs side) {
    if (blockIdx.x < side.groups) {
        const uint64_t tb = side.gate->tile_bytes;
        if (__builtin_amdgcn_readfirstlane((uint32_t)(side.any_tile | (tb == a.tile_bytes))))
            side_part<THREADS>(side, blockIdx.x);
        return;
    }
    move_launch_tiles<THREADS, VPT, NT>(a, blockIdx.x - side.groups);
}

template <int THREADS, int VPT, int NT>
hipError_t launch_t(const MoveArgs &a, uint32_t wg_per_cu, int num_cus, hipStream_t s) {
    const size_t lds = (size_t)a.max_blocks * 12u + 16u;
    uint64_t per_cu = wg_per_cu;
    if (per_cu == 0) {  // as many as the kernel's resources allow (the query costs a few us)
        int occ = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, k_move<THREADS, VPT, NT>, THREADS, lds);
        if (e != hipSuccess) return e;
        per_cu = occ < 1 ? 1u : (uint32_t)occ;
    }
    uint64_t grid = per_cu * (uint64_t)num_cus;
    if (grid > a.n_tiles) grid = a.n_tiles;
    if (grid > kMaxMoveGrid) grid = kMaxMoveGrid;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((k_move<THREADS, VPT, NT>), dim3((uint32_t)grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

// The device-sized mover: the grid the plan's tuning asks for (the plan is
// not read back first: the workgroups read its tile count from the device),
// LDS for the most blocks a tile can meet.
template <int THREADS, int VPT, int NT>
hipError_t launch_device_sized_t(const MoveArgs &a, const SideArgs *side, hipStream_t s) {
    const size_t lds = (size_t)a.max_blocks * 12u + 16u;
    const uint64_t per_cu = a.wg_per_cu ? a.wg_per_cu : kDefaultWgPerCu;
    uint64_t grid = per_cu * (uint64_t)a.num_cus;
    if (grid > kMaxMoveGrid) grid = kMaxMoveGrid;
    if (grid < 1) grid = 1;
    if (side) {
        if (!side->gate) return hipErrorInvalidValue;  // the job reads the plan's header
        SideArgs sj = *side;
        size_side(sj, THREADS, (int)a.num_cus);
        hipLaunchKernelGGL((k_move_side<THREADS, VPT, NT>), dim3((uint32_t)(grid + sj.groups)),
                           dim3(THREADS), lds, s, a, sj);
    } else {
        hipLaunchKernelGGL((k_move<THREADS, VPT, NT>), dim3((uint32_t)grid), dim3(THREADS), lds,
                           s, a);
    }
    return hipGetLastError();
}

template <int THREADS, int VPT, int NT, bool DEVICE_SIZED>
hipError_t launch_one(const MoveArgs &a, uint32_t wg_per_cu, int num_cus, const SideArgs *side,
                      hipStream_t s) {
    if constexpr (VPT * THREADS * 16 > kMaxTile) {
        return hipErrorInvalidValue;  // larger than any tile
    } else if constexpr (DEVICE_SIZED) {
        return launch_device_sized_t<THREADS, VPT, NT>(a, side, s);
    } else {
        return launch_t<THREADS, VPT, NT>(a, wg_per_cu, num_cus, s);
    }
}

// Vectors per lane: the tile over the workgroup's row of 16-byte vectors.
template <int THREADS, int NT, bool DEVICE_SIZED>
hipError_t launch_threads(const MoveArgs &a, uint32_t wg_per_cu, int num_cus,
                          const SideArgs *side, hipStream_t s) {
    constexpr uint32_t row = THREADS * 16;
    switch (a.tile_bytes <= row ? 1u : a.tile_bytes / row) {
        case 1: return launch_one<THREADS, 1, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus, side, s);
        case 2: return launch_one<THREADS, 2, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus, side, s);
        case 4: return launch_one<THREADS, 4, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus, side, s);
        case 8: return launch_one<THREADS, 8, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus, side, s);
        case 16: return launch_one<THREADS, 16, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus, side, s);
        case 32: return launch_one<THREADS, 32, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus, side, s);
        default: return hipErrorInvalidValue;
    }
}

template <int NT, bool DEVICE_SIZED>
hipError_t launch_nt(const MoveArgs &a, uint32_t wg_per_cu, int num_cus, const SideArgs *side,
                     hipStream_t s) {
    return a.small_blocks ? launch_threads<kMoveThreadsSmallBlocks, NT, DEVICE_SIZED>(
                                a, wg_per_cu, num_cus, side, s)
                          : launch_threads<kMoveThreads, NT, DEVICE_SIZED>(a, wg_per_cu, num_cus,
                                                                          side, s);
}

}  // namespace

hipError_t launch_move(const MoveArgs &a, uint32_t wg_per_cu, uint32_t nontemporal, int num_cus,
                       hipStream_t s) {
    if (a.n_tiles == 0) return hipSuccess;
    uint64_t vgrid = (a.n_tiles + 255) / 256;
    if (vgrid > (uint64_t)num_cus * 4) vgrid = (uint64_t)num_cus * 4;
    hipLaunchKernelGGL(k_verify_tiles, dim3((uint32_t)vgrid), dim3(256), 0, s, a);
    AC_TRY(hipGetLastError());
    switch (nontemporal) {
        case 0: return launch_nt<0, false>(a, wg_per_cu, num_cus, nullptr, s);
        case 1: return launch_nt<3, false>(a, wg_per_cu, num_cus, nullptr, s);
        case 2: return launch_nt<1, false>(a, wg_per_cu, num_cus, nullptr, s);
        case 3: return launch_nt<2, false>(a, wg_per_cu, num_cus, nullptr, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_move_device_sized(const MoveArgs &a, uint32_t nontemporal,
                                    const SideArgs *side, hipStream_t s) {
    switch (nontemporal) {
        case 0: return launch_nt<0, true>(a, 0, 0, side, s);
        case 1: return launch_nt<3, true>(a, 0, 0, side, s);
        case 2: return launch_nt<1, true>(a, 0, 0, side, s);
        case 3: return launch_nt<2, true>(a, 0, 0, side, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ac

// plan.hip -- validation, live-size scan, hole statistics and the mover's tile
// table, for gfx950 (wave64).
//
// Page: "Ascend 910C cluster tuning: memory-fragment compaction in
// mixed-precision training", section "Periodic compaction with Ascend C":
// holes are scanned from low to high addresses and each live tensor gets the
// downward shift it needs.  Here that is an exclusive scan over the table of
// the triple (live size, live end, live count):
//   new offset of entry i   = sum of live sizes before i
//   hole just below live i  = offset_i - (end of the previous live block)
//                           = offset_i - max of live ends before i
//   index of i among live   = count of live entries before i
// Section "Total-usage monitoring misses fragmentation" of the same page asks
// for the free total and the largest contiguous free block; section 3.2 of
// "CANN memory management and memory optimisation" defines the ratio
// 1 - largest/free.  Holes are maximal runs outside live blocks (the CANN pool
// merges adjacent free blocks, section 2.2), so one pass over live entries in
// order sees every hole once, plus the tail above the highest live block.
//
// Three passes (n up to 2^32 entries): per-workgroup aggregates, a
// single-workgroup spine scan of the aggregates, then a downsweep that writes
// new offsets, the packed live-block arrays and per-workgroup hole/move
// statistics, reduced by a final single-workgroup pass.  Table traffic is
// 17 B per entry read twice plus 8 B per entry of new offsets and 16 B per
// live block written.
#include "internal.h"

namespace ac {
namespace {

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Reason code of entry i (0 when it passes); checks in the documented order.
__device__ inline uint32_t entry_reason(uint64_t i, uint64_t o, uint64_t s, uint32_t l,
                                        uint64_t arena_bytes, uint64_t prev_end) {
    if (s == 0) return 1;
    if ((o | s) & 31u) return 2;
    if (l > 1u) return 3;
    if (o > arena_bytes || s > arena_bytes - o) return 4;
    if (i > 0 && prev_end > o) return 5;
    return 0;
}

// Inclusive wave64 scan of (a: sum, b: max, c: sum).
__device__ inline void wave_incl_scan3(uint64_t &a, uint64_t &b, uint64_t &c) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t ya = __shfl_up(a, d, 64);
        const uint64_t yb = __shfl_up(b, d, 64);
        const uint64_t yc = __shfl_up(c, d, 64);
        if (lane >= d) {
            a += ya;
            b = umax64(b, yb);
            c += yc;
        }
    }
}

// Exclusive workgroup scan of (a, b, c) with identity (0, 0, 0); also returns
// the workgroup totals.  sh needs 3 * NT/64 entries.
template <int NT>
__device__ inline void block_excl_scan3(uint64_t &a, uint64_t &b, uint64_t &c,
                                        uint64_t &ta, uint64_t &tb, uint64_t &tc,
                                        uint64_t *sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    uint64_t ia = a, ib = b, ic = c;
    wave_incl_scan3(ia, ib, ic);
    if (lane == 63) {
        sh[w] = ia;
        sh[NW + w] = ib;
        sh[2 * NW + w] = ic;
    }
    __syncthreads();
    uint64_t pa = 0, pb = 0, pc = 0;
    ta = 0;
    tb = 0;
    tc = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const uint64_t xa = sh[k], xb = sh[NW + k], xc = sh[2 * NW + k];
        if (k < w) {
            pa += xa;
            pb = umax64(pb, xb);
            pc += xc;
        }
        ta += xa;
        tb = umax64(tb, xb);
        tc += xc;
    }
    uint64_t ea = __shfl_up(ia, 1, 64), eb = __shfl_up(ib, 1, 64), ec = __shfl_up(ic, 1, 64);
    if (lane == 0) {
        ea = 0;
        eb = 0;
        ec = 0;
    }
    a = pa + ea;
    b = umax64(pb, eb);
    c = pc + ec;
    __syncthreads();
}

// Workgroup reductions through LDS (NT threads, sh has NT/64 slots).
template <int NT, typename Op>
__device__ inline uint64_t block_reduce(uint64_t v, uint64_t *sh, Op op) {
    constexpr int NW = NT / 64;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = op(v, (uint64_t)__shfl_xor(v, d, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = sh[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) r = op(r, sh[k]);
    __syncthreads();
    return r;
}

struct OpAdd { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; } };
struct OpMax { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return umax64(a, b); } };
struct OpMin { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return umin64(a, b); } };

// Pass 1: per-workgroup (live size sum, live end max, live count, first bad key).
__global__ __launch_bounds__(kScanThreads) void k_scan_partials(TableView t, uint64_t arena_bytes,
                                                                ScanPart *part) {
    __shared__ uint64_t sh[kScanThreads / 64];
    const uint64_t i0 = (uint64_t)blockIdx.x * kScanTile + (uint64_t)threadIdx.x * kScanItems;
    uint64_t sum = 0, mx = 0, cnt = 0, bad = kNone;
    uint64_t prev_end = 0;
    if (i0 > 0 && i0 < t.n) prev_end = t.off[i0 - 1] + t.size[i0 - 1];
#pragma unroll
    for (uint32_t k = 0; k < kScanItems; ++k) {
        const uint64_t i = i0 + k;
        if (i < t.n) {
            const uint64_t o = t.off[i], s = t.size[i];
            const uint32_t l = t.live ? t.live[i] : 1u;
            const uint32_t r = entry_reason(i, o, s, l, arena_bytes, prev_end);
            if (r) bad = umin64(bad, (i << 3) | r);
            if (l) {
                sum += s;
                mx = umax64(mx, o + s);
                cnt += 1;
            }
            prev_end = o + s;
        }
    }
    sum = block_reduce<kScanThreads>(sum, sh, OpAdd());
    mx = block_reduce<kScanThreads>(mx, sh, OpMax());
    cnt = block_reduce<kScanThreads>(cnt, sh, OpAdd());
    bad = block_reduce<kScanThreads>(bad, sh, OpMin());
    if (threadIdx.x == 0) part[blockIdx.x] = ScanPart{sum, mx, cnt, bad};
}

// Pass 2 (one workgroup): exclusive scan of the aggregates; table totals.
__global__ __launch_bounds__(kSpineThreads) void k_scan_spine(const ScanPart *part, ScanPart *prefix,
                                                              uint64_t nb, WsHeader *hdr) {
    __shared__ uint64_t sh[3 * kSpineThreads / 64];
    __shared__ uint64_t shr[kSpineThreads / 64];
    uint64_t ca = 0, cb = 0, cc = 0, bad = kNone;
    for (uint64_t base = 0; base < nb; base += kSpineThreads) {
        const uint64_t j = base + threadIdx.x;
        uint64_t a = 0, b = 0, c = 0;
        if (j < nb) {
            const ScanPart p = part[j];
            a = p.sum;
            b = p.maxend;
            c = p.count;
            bad = umin64(bad, p.bad_key);
        }
        uint64_t ta, tb, tc;
        block_excl_scan3<kSpineThreads>(a, b, c, ta, tb, tc, sh);
        if (j < nb) prefix[j] = ScanPart{ca + a, umax64(cb, b), cc + c, 0};
        ca += ta;
        cb = umax64(cb, tb);
        cc += tc;
    }
    bad = block_reduce<kSpineThreads>(bad, shr, OpMin());
    if (threadIdx.x == 0) {
        hdr->live_bytes = ca;
        hdr->max_live_end = cb;
        hdr->live_blocks = cc;
        hdr->bad_key = bad;
    }
}

// Pass 3: new offsets, packed live arrays, per-workgroup hole/move stats.
__global__ __launch_bounds__(kScanThreads) void k_scan_down(TableView t, const ScanPart *prefix,
                                                            const WsHeader *hdr, uint64_t *new_offset,
                                                            uint64_t *live_dst, uint64_t *live_src,
                                                            StatPart *spart, int write_outputs) {
    __shared__ uint64_t sh[3 * kScanThreads / 64];
    if (hdr->bad_key != kNone) return;  // invalid table: write nothing
    const uint64_t i0 = (uint64_t)blockIdx.x * kScanTile + (uint64_t)threadIdx.x * kScanItems;
    uint64_t o[kScanItems], s[kScanItems];
    uint32_t l[kScanItems];
    uint64_t a = 0, b = 0, c = 0;
#pragma unroll
    for (uint32_t k = 0; k < kScanItems; ++k) {
        const uint64_t i = i0 + k;
        o[k] = 0;
        s[k] = 0;
        l[k] = 0;
        if (i < t.n) {
            o[k] = t.off[i];
            s[k] = t.size[i];
            l[k] = t.live ? t.live[i] : 1u;
            if (l[k]) {
                a += s[k];
                b = umax64(b, o[k] + s[k]);
                c += 1;
            }
        }
    }
    uint64_t ta, tb, tc;
    block_excl_scan3<kScanThreads>(a, b, c, ta, tb, tc, sh);
    const ScanPart P = prefix[blockIdx.x];
    uint64_t run_sum = P.sum + a;
    uint64_t run_end = umax64(P.maxend, b);
    uint64_t run_cnt = P.count + c;
    uint64_t max_gap = 0, gaps = 0, moved = 0, moved_bytes = 0, first_moved = kNone,
             min_size = kNone;
#pragma unroll
    for (uint32_t k = 0; k < kScanItems; ++k) {
        const uint64_t i = i0 + k;
        if (i < t.n) {
            if (write_outputs && new_offset) new_offset[i] = run_sum;
            if (l[k]) {
                if (write_outputs) {
                    live_dst[run_cnt] = run_sum;
                    live_src[run_cnt] = o[k];
                }
                const uint64_t gap = o[k] - run_end;
                if (gap) {
                    gaps += 1;
                    max_gap = umax64(max_gap, gap);
                }
                if (o[k] != run_sum) {
                    moved += 1;
                    moved_bytes += s[k];
                    first_moved = umin64(first_moved, run_cnt);
                }
                min_size = umin64(min_size, s[k]);
                run_sum += s[k];
                run_end = o[k] + s[k];
                run_cnt += 1;
            }
        }
    }
    max_gap = block_reduce<kScanThreads>(max_gap, sh, OpMax());
    gaps = block_reduce<kScanThreads>(gaps, sh, OpAdd());
    moved = block_reduce<kScanThreads>(moved, sh, OpAdd());
    moved_bytes = block_reduce<kScanThreads>(moved_bytes, sh, OpAdd());
    first_moved = block_reduce<kScanThreads>(first_moved, sh, OpMin());
    min_size = block_reduce<kScanThreads>(min_size, sh, OpMin());
    if (threadIdx.x == 0)
        spart[blockIdx.x] = StatPart{max_gap, gaps, moved, moved_bytes, first_moved, min_size, {0, 0}};
}

// Pass 4 (one workgroup): reduce the statistics, add the tail hole, and set
// the move range.
__global__ __launch_bounds__(kSpineThreads) void k_scan_finish(const StatPart *spart, uint64_t nb,
                                                               uint64_t arena_bytes, WsHeader *hdr,
                                                               uint64_t *live_dst, uint64_t *live_src,
                                                               int write_outputs, uint64_t epoch) {
    __shared__ uint64_t sh[kSpineThreads / 64];
    if (hdr->bad_key != kNone) return;
    uint64_t max_gap = 0, gaps = 0, moved = 0, moved_bytes = 0, first_moved = kNone,
             min_size = kNone;
    for (uint64_t j = threadIdx.x; j < nb; j += kSpineThreads) {
        const StatPart p = spart[j];
        max_gap = umax64(max_gap, p.max_gap);
        gaps += p.gaps;
        moved += p.moved_blocks;
        moved_bytes += p.moved_bytes;
        first_moved = umin64(first_moved, p.first_moved);
        min_size = umin64(min_size, p.min_size);
    }
    max_gap = block_reduce<kSpineThreads>(max_gap, sh, OpMax());
    gaps = block_reduce<kSpineThreads>(gaps, sh, OpAdd());
    moved = block_reduce<kSpineThreads>(moved, sh, OpAdd());
    moved_bytes = block_reduce<kSpineThreads>(moved_bytes, sh, OpAdd());
    first_moved = block_reduce<kSpineThreads>(first_moved, sh, OpMin());
    min_size = block_reduce<kSpineThreads>(min_size, sh, OpMin());
    if (threadIdx.x == 0) {
        const uint64_t m = hdr->live_blocks;
        const uint64_t lt = hdr->live_bytes;
        const uint64_t tail = arena_bytes - hdr->max_live_end;
        hdr->largest_hole = umax64(max_gap, tail);
        hdr->hole_count = gaps + (tail ? 1 : 0);
        hdr->moved_blocks = moved;
        hdr->moved_bytes = moved_bytes;
        hdr->first_moved = first_moved == kNone ? m : first_moved;
        hdr->min_live_size = min_size;
        // plan fields: a statistics-only pass leaves an existing plan intact
        if (write_outputs) {
            live_dst[m] = lt;
            live_src[m] = arena_bytes;
            hdr->move_begin = first_moved != kNone ? live_dst[first_moved] : lt;
            hdr->epoch = epoch;
            hdr->ticket = 0;
            hdr->status = 0;
        }
    }
}

// Largest k in [lo, hi) with a[k] <= x, or lo - 1 if none (as int64).
__device__ inline int64_t last_le(const uint64_t *a, int64_t lo, int64_t hi, uint64_t x) {
    int64_t l = lo, h = hi;  // find first index with a[k] > x in [lo, hi)
    while (l < h) {
        const int64_t mid = l + ((h - l) >> 1);
        if (a[mid] <= x) l = mid + 1;
        else h = mid;
    }
    return l - 1;
}

// Tile table: one thread per destination tile.  Tile t covers destination
// bytes [max(base + tT, begin), min(base + (t+1)T, LT)).  The move writes
// p from p + shift(p); a tile may only write once every tile whose source
// range overlaps its destination has read.  Sources move strictly upward
// with destinations, so those sources come from one destination interval no
// longer than T: at most two tiles, both at or below t.
__global__ __launch_bounds__(256) void k_tiles(const uint64_t *live_dst, const uint64_t *live_src,
                                               TileRec *tiles, uint32_t *flags, uint64_t n_tiles,
                                               uint64_t base, uint64_t T, uint64_t begin, uint64_t lt,
                                               uint64_t k0, uint64_t m) {
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_tiles) return;
    const uint64_t tb = base + t * T;
    const uint64_t t0 = umax64(tb, begin);
    const uint64_t t1 = umin64(tb + T, lt);
    const int64_t first = last_le(live_dst, (int64_t)k0, (int64_t)m, t0);
    const int64_t last = last_le(live_dst, (int64_t)k0, (int64_t)m, t1 - 1);
    // first moved block whose source ends above t0
    int64_t l = (int64_t)k0, h = (int64_t)m;
    while (l < h) {
        const int64_t mid = l + ((h - l) >> 1);
        const uint64_t src_end = live_src[mid] + (live_dst[mid + 1] - live_dst[mid]);
        if (src_end <= t0) l = mid + 1;
        else h = mid;
    }
    uint32_t dep_lo = 1, dep_hi = 0;  // empty
    if (l < (int64_t)m && live_src[l] < t1 && t > 0) {
        const uint64_t j = (uint64_t)l;
        const uint64_t q_lo = live_dst[j] + (t0 > live_src[j] ? t0 - live_src[j] : 0);
        const int64_t c = last_le(live_src, (int64_t)j, (int64_t)m, t1 - 1);
        const uint64_t cs = live_dst[c + 1] - live_dst[c];
        const uint64_t q_hi = live_dst[c] + umin64(cs, t1 - live_src[c]) - 1;
        const uint64_t lo_t = (q_lo - base) / T;
        uint64_t hi_t = (q_hi - base) / T;
        if (hi_t > t - 1) hi_t = t - 1;
        if (lo_t <= hi_t) {
            dep_lo = (uint32_t)lo_t;
            dep_hi = (uint32_t)hi_t;
        }
    }
    tiles[t] = TileRec{(uint32_t)first, (uint32_t)last, dep_lo, dep_hi};
    flags[t] = 0u;
}

__global__ void k_commit(const uint64_t *live_dst, uint64_t m, uint64_t *off_out,
                         uint64_t *size_out, uint8_t *live_out) {
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < m;
         k += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t d = live_dst[k];
        if (off_out) off_out[k] = d;
        if (size_out) size_out[k] = live_dst[k + 1] - d;
        if (live_out) live_out[k] = 1;
    }
}

}  // namespace

hipError_t launch_scan(const TableView &t, uint64_t arena_bytes, uint8_t *ws, const WsLayout &L,
                       uint64_t *new_offset, bool write_outputs, uint64_t epoch, hipStream_t s) {
    WsHeader *hdr = reinterpret_cast<WsHeader *>(ws + L.header);
    ScanPart *part = reinterpret_cast<ScanPart *>(ws + L.part);
    ScanPart *prefix = reinterpret_cast<ScanPart *>(ws + L.prefix);
    StatPart *spart = reinterpret_cast<StatPart *>(ws + L.spart);
    uint64_t *live_dst = reinterpret_cast<uint64_t *>(ws + L.live_dst);
    uint64_t *live_src = reinterpret_cast<uint64_t *>(ws + L.live_src);
    const uint64_t nb = L.n_scan_blocks;
    if (nb) {
        hipLaunchKernelGGL(k_scan_partials, dim3((uint32_t)nb), dim3(kScanThreads), 0, s, t,
                           arena_bytes, part);
    }
    hipLaunchKernelGGL(k_scan_spine, dim3(1), dim3(kSpineThreads), 0, s, part, prefix, nb, hdr);
    if (nb) {
        hipLaunchKernelGGL(k_scan_down, dim3((uint32_t)nb), dim3(kScanThreads), 0, s, t, prefix,
                           hdr, new_offset, live_dst, live_src, spart, write_outputs ? 1 : 0);
    }
    hipLaunchKernelGGL(k_scan_finish, dim3(1), dim3(kSpineThreads), 0, s, spart, nb, arena_bytes,
                       hdr, live_dst, live_src, write_outputs ? 1 : 0, epoch);
    return hipGetLastError();
}

hipError_t launch_tiles(uint8_t *ws, const WsLayout &L, uint64_t n_tiles, uint64_t tile_base,
                        uint32_t tile_bytes, uint64_t move_begin, uint64_t live_bytes,
                        uint64_t first_moved, uint64_t live_blocks, hipStream_t s) {
    if (n_tiles == 0) return hipSuccess;
    const uint64_t *live_dst = reinterpret_cast<const uint64_t *>(ws + L.live_dst);
    const uint64_t *live_src = reinterpret_cast<const uint64_t *>(ws + L.live_src);
    TileRec *tiles = reinterpret_cast<TileRec *>(ws + L.tiles);
    uint32_t *flags = reinterpret_cast<uint32_t *>(ws + L.flags);
    const uint64_t grid = (n_tiles + 255) / 256;
    hipLaunchKernelGGL(k_tiles, dim3((uint32_t)grid), dim3(256), 0, s, live_dst, live_src, tiles,
                       flags, n_tiles, tile_base, (uint64_t)tile_bytes, move_begin, live_bytes,
                       first_moved, live_blocks);
    return hipGetLastError();
}

hipError_t launch_commit(const uint8_t *ws, const WsLayout &L, uint64_t live_blocks,
                         uint64_t *off_out, uint64_t *size_out, uint8_t *live_out, hipStream_t s) {
    if (live_blocks == 0) return hipSuccess;
    const uint64_t *live_dst = reinterpret_cast<const uint64_t *>(ws + L.live_dst);
    uint64_t grid = (live_blocks + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_commit, dim3((uint32_t)grid), dim3(256), 0, s, live_dst, live_blocks,
                       off_out, size_out, live_out);
    return hipGetLastError();
}

}  // namespace ac

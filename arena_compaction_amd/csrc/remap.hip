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
// One lane per handle, grid-stride.  The search runs over the plan's packed
// live-block arrays (old offsets ascending, and new offsets whose successive
// differences are the block sizes), so free entries never cost a probe.  The
// search is branchless with a trip count fixed by the table size, so the 64
// lanes of a wave step together.  HBM traffic is 16 B per handle; the probes
// hit the top of the table, which stays in L2 and the Infinity Cache.
#include "internal.h"

namespace ac {
namespace {

__global__ __launch_bounds__(256) void k_remap(const uint64_t *__restrict__ live_dst,
                                               const uint64_t *__restrict__ live_src, uint64_t m,
                                               const uint64_t *h_in, uint64_t *h_out, uint64_t H,
                                               unsigned long long *n_invalid) {
    uint64_t bad = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < H; k += stride) {
        const uint64_t h = h_in[k];
        uint64_t out = kNone;
        if (m) {
            // largest j with live_src[j] <= h (j = 0 when none; checked below)
            uint64_t lo = 0, n = m;
            while (n > 1) {
                const uint64_t half = n >> 1;
                lo = (live_src[lo + half] <= h) ? lo + half : lo;
                n -= half;
            }
            const uint64_t src = live_src[lo];
            if (src <= h) {
                const uint64_t d = live_dst[lo];
                const uint64_t size = live_dst[lo + 1] - d;
                if (h - src < size) out = d + (h - src);
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

__global__ void k_zero_u64(uint64_t *p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

}  // namespace

hipError_t launch_remap(const uint64_t *live_dst, const uint64_t *live_src, uint64_t live_blocks,
                        const uint64_t *h_in, uint64_t *h_out, uint64_t n_handles,
                        uint64_t *n_invalid, int num_cus, hipStream_t s) {
    if (n_invalid) hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, s, n_invalid);
    if (n_handles == 0) return hipGetLastError();
    uint64_t grid = (n_handles + 255) / 256;
    const uint64_t cap = (uint64_t)num_cus * 16;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(k_remap, dim3((uint32_t)grid), dim3(256), 0, s, live_dst, live_src,
                       live_blocks, h_in, h_out, n_handles,
                       reinterpret_cast<unsigned long long *>(n_invalid));
    return hipGetLastError();
}

}  // namespace ac

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
// live-block arrays (old offsets ascending, new offsets, sizes), so free
// entries never cost a probe; a pinned block maps to itself.  A
// plain binary search is bound by L2 transactions (every probe of every lane
// is its own cache line), so the top levels run in LDS over a sample of the
// old offsets and only the last few probe global memory.  HBM traffic is
// 16 B per handle.
#include "internal.h"

namespace ac {
namespace {

constexpr uint32_t kRemapThreads = 256;
constexpr uint32_t kSplitters = 4096;  // 32 KB of LDS per workgroup

// Largest j in [lo, lo + n) with a[j] <= h, given a[lo] <= h (or j = lo).
template <typename T>
__device__ __forceinline__ uint64_t search_le(const T *a, uint64_t lo, uint64_t n, uint64_t h) {
    while (n > 1) {
        const uint64_t half = n >> 1;
        lo = ((uint64_t)a[lo + half] <= h) ? lo + half : lo;
        n -= half;
    }
    return lo;
}

// The top of each search runs in LDS over a sample of every step-th old
// offset; the rest runs over one bucket of at most `step` offsets in global
// memory (L2-resident).  For m <= kSplitters the sample is the whole array.
// Searches are branchless with trip counts set by the sizes alone, so the
// 64 lanes of a wave step together.
__global__ __launch_bounds__(kRemapThreads) void k_remap(const uint64_t *__restrict__ live_dst,
                                                         const uint64_t *__restrict__ live_src,
                                                         const uint64_t *__restrict__ live_size,
                                                         uint64_t m, const uint64_t *h_in,
                                                         uint64_t *h_out, uint64_t H,
                                                         unsigned long long *n_invalid) {
    __shared__ uint64_t sp[kSplitters];
    const uint64_t step = (m + kSplitters - 1) / kSplitters;
    const uint64_t ns = m ? (m + step - 1) / step : 0;
    for (uint64_t i = threadIdx.x; i < ns; i += kRemapThreads) sp[i] = live_src[i * step];
    __syncthreads();
    uint64_t bad = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < H; k += stride) {
        const uint64_t h = h_in[k];
        uint64_t out = kNone;
        if (ns && sp[0] <= h) {
            const uint64_t b = search_le(sp, 0, ns, h);
            const uint64_t lo = b * step;
            const uint64_t hi = (lo + step < m) ? lo + step : m;
            const uint64_t j = search_le(live_src, lo, hi - lo, h);
            const uint64_t src = live_src[j];
            if (h - src < live_size[j]) out = live_dst[j] + (h - src);
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

hipError_t launch_remap(const LiveView &lv, uint64_t live_blocks, const uint64_t *h_in,
                        uint64_t *h_out, uint64_t n_handles, uint64_t *n_invalid, int num_cus,
                        hipStream_t s) {
    if (n_invalid) hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, s, n_invalid);
    if (n_handles == 0) return hipGetLastError();
    // persistent grid: every workgroup pays for loading the LDS sample once
    uint64_t grid = (n_handles + kRemapThreads - 1) / kRemapThreads;
    const uint64_t cap = (uint64_t)num_cus * 4;  // measured best of 4, 5 and 8 per CU
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(k_remap, dim3((uint32_t)grid), dim3(kRemapThreads), 0, s, lv.dst, lv.src,
                       lv.size, live_blocks, h_in, h_out, n_handles,
                       reinterpret_cast<unsigned long long *>(n_invalid));
    return hipGetLastError();
}

}  // namespace ac

// publish.hip -- the device half of a read-back: a one-wave kernel that
// copies a result header into a pinned, device-mapped host slot and then
// stores the read-back's sequence number there with system-scope release,
// so the host that sees the number sees the header.  Every store is a
// per-lane vector store to the slot.
#include "internal.h"

namespace ac {
namespace {

__global__ __launch_bounds__(64) void k_publish(const uint64_t *__restrict__ src,
                                                uint64_t *__restrict__ dst, uint32_t words,
                                                uint64_t *seq_out, uint64_t seq) {
    for (uint32_t i = threadIdx.x; i < words; i += 64) dst[i] = src[i];
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(seq_out, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

hipError_t launch_publish(const uint64_t *src, uint64_t *dst_host, uint32_t words,
                          uint64_t *seq_host, uint64_t seq, hipStream_t s) {
    hipLaunchKernelGGL(k_publish, dim3(1), dim3(64), 0, s, src, dst_host, words, seq_host, seq);
    return hipGetLastError();
}

}  // namespace ac

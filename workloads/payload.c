/* Host-side payload generator: the same counter-based functions as the torch
 * code in workloads/__init__.py, for CPU buffers (the torch path serves GPU
 * tensors).  Input generation only -- nothing of the compactor is here.
 *
 *   hash      : 8-byte word w = output w of SplitMix64 seeded with `seed`
 *               (Steele, Lea & Flood, OOPSLA 2014): the state advances by the
 *               golden gamma before each output, then the 64-bit finaliser.
 *   counter32 : 4-byte word j = (j mod 2^32) XOR seed.
 */
#include <stdint.h>
#include <string.h>

static inline uint64_t sm64_out(uint64_t seed, uint64_t k) {
    uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* dst receives words [w0, w0 + count) */
void wl_fill_hash(uint8_t *dst, uint64_t w0, uint64_t count, uint64_t seed) {
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < (int64_t)count; ++k) {
        const uint64_t v = sm64_out(seed, w0 + (uint64_t)k);
        memcpy(dst + 8 * k, &v, 8);
    }
}

void wl_fill_counter32(uint8_t *dst, uint64_t j0, uint64_t count, uint32_t seed) {
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < (int64_t)count; ++k) {
        const uint32_t v = (uint32_t)(j0 + (uint64_t)k) ^ seed;
        memcpy(dst + 4 * k, &v, 4);
    }
}

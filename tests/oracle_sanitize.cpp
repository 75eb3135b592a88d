// Runs every oracle function over many random small tables, with checks
// that tie them together, so that a build with AddressSanitizer and
// UndefinedBehaviorSanitizer exercises all of the oracle's code.  Built and
// run by tests/test_oracle_sanitize.py on the CPU; exits non-zero on a
// failed check (the sanitizers abort on their own findings).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../oracle/oracle.h"

namespace {

int failures = 0;

void check(bool ok, const char *what, int iter) {
    if (!ok) {
        std::fprintf(stderr, "check failed: %s (table %d)\n", what, iter);
        ++failures;
    }
}

}  // namespace

int main() {
    std::mt19937_64 rng(12345);
    for (int iter = 0; iter < 4000; ++iter) {
        const uint64_t n = rng() % 24;
        std::vector<uint64_t> off(n), size(n);
        std::vector<uint8_t> live(n), pin(n);
        uint64_t cur = 0;
        for (uint64_t i = 0; i < n; ++i) {
            cur += 32 * (rng() % 3 == 0 ? rng() % 4 : 0);
            off[i] = cur;
            size[i] = 32 * (1 + rng() % 6);
            cur += size[i];
            live[i] = rng() % 3 != 0;
            pin[i] = live[i] && rng() % 5 == 0;
        }
        const uint64_t S = cur + 32 * (rng() % 3) + (rng() % 2 ? rng() % 32 : 0);
        const uint8_t *pinned = (iter % 2) ? pin.data() : nullptr;

        uint64_t bad = 0;
        int32_t reason = 0;
        check(oracle_validate(off.data(), size.data(), live.data(), pinned, n, S, &bad,
                              &reason) == ORACLE_OK, "valid table", iter);

        std::vector<uint64_t> nw(n);
        oracle_new_offsets(off.data(), size.data(), live.data(), pinned, n, nw.data());

        oracle_stats st;
        oracle_stats_walk(off.data(), size.data(), live.data(), pinned, n, S, &st);
        check(st.free_bytes + st.live_bytes == S, "free + live = arena", iter);

        std::vector<uint8_t> arena(S), ref(S);
        for (uint64_t p = 0; p < S; ++p) arena[p] = (uint8_t)(rng() & 255);
        ref = arena;
        oracle_compact(arena.data(), S, off.data(), size.data(), live.data(), pinned, n);
        // every live block's bytes at its new place
        for (uint64_t i = 0; i < n; ++i)
            if (live[i])
                check(std::memcmp(arena.data() + nw[i], ref.data() + off[i], size[i]) == 0,
                      "payload at new offset", iter);
        // the source map rebuilds the whole compacted arena
        std::vector<uint64_t> d(4 * n + 4), s(4 * n + 4), l(4 * n + 4);
        const int64_t k = oracle_source_map(off.data(), size.data(), live.data(), pinned, n, S,
                                            0, S, d.data(), s.data(), l.data(), d.size());
        check(k >= 0, "source map fits", iter);
        for (int64_t q = 0; q < k; ++q)
            check(std::memcmp(arena.data() + d[q], ref.data() + s[q], l[q]) == 0,
                  "source map piece", iter);

        // remap: every byte of every live block, plus handles past the end
        std::vector<uint64_t> h, hout;
        for (uint64_t i = 0; i < n; ++i)
            for (uint64_t b = 0; b < size[i]; b += 16) h.push_back(off[i] + b);
        h.push_back(S);
        h.push_back(S + 1000);
        h.push_back(UINT64_MAX);
        hout.resize(h.size());
        uint64_t n_bad = 0;
        oracle_remap(off.data(), size.data(), live.data(), pinned, n, h.data(), hout.data(),
                     h.size(), &n_bad);
        for (size_t q = 0; q < h.size(); ++q)
            if (hout[q] != UINT64_MAX) check(arena[hout[q]] == ref[h[q]], "remapped byte", iter);

        // targeted window, first fit and monitor on the same table
        for (uint64_t R : {uint64_t(1), uint64_t(32), uint64_t(96), S / 2 + 1, S, S + 1}) {
            if (R == 0) continue;
            oracle_window w;
            check(oracle_target_window(off.data(), size.data(), live.data(), pinned, n, S, R,
                                       &w) == ORACLE_OK, "window call", iter);
            if (w.found) check(w.hole >= R && w.end <= S && w.begin <= w.end, "window", iter);
            uint64_t ff = 0;
            check(oracle_first_fit(off.data(), size.data(), live.data(), n, S, R, &ff) ==
                      ORACLE_OK, "first fit call", iter);
            if (ff != UINT64_MAX) check(ff < S, "first fit inside", iter);
            oracle_monitor_out mo;
            oracle_monitor(S, st.live_bytes, st.largest_hole, 0.85, 0.95, 1.0, R, 1e6, &mo);
            check(mo.level >= 0 && mo.level <= 2 && mo.action >= 0 && mo.action <= 3,
                  "monitor ranges", iter);
        }
    }
    // invalid tables: every reason path
    {
        const uint64_t off[3] = {0, 16, 64}, size[3] = {32, 32, 0};
        const uint8_t live[3] = {1, 2, 1};
        uint64_t bad = 0;
        int32_t reason = 0;
        check(oracle_validate(off, size, live, nullptr, 3, 64, &bad, &reason) == ORACLE_EINVAL,
              "invalid table", -1);
    }
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("oracle sanitize run ok\n");
    return 0;
}

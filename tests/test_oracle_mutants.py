"""The oracle's pins must catch plausible mistakes.  Each case below plants
one mistake in a copy of oracle.cpp (a dropped term, a swapped operand, an
off-by-one, a wrong order), builds it, and checks that the pin battery of
tests/test_oracle.py rejects it.  Mistakes are planted on the CPU only."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import workloads as W
import test_oracle as T
import test_oracle_targeted as TT
import test_oracle_first_fit as FF
import test_oracle_monitor as MO

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

# (name, exact text in oracle.cpp, replacement)
MUTANTS = [
    ("scan_inclusive", "        new_offset[i] = running;\n        if (live[i]) running += size[i];",
     "        if (live[i]) running += size[i];\n        new_offset[i] = running;"),
    ("scan_ignores_live", "        if (live[i]) running += size[i];", "        running += size[i];"),
    ("compact_moves_free", "        if (!live[i]) continue;\n        if (dst != offset[i])",
     "        if (live[i]) continue;\n        if (dst != offset[i])"),
    ("ratio1_transposed", "out->frag_free_over_largest_minus_1 = F / L - 1.0;",
     "out->frag_free_over_largest_minus_1 = L / F - 1.0;"),
    ("ratio2_transposed", "out->frag_one_minus_largest_over_free = 1.0 - L / F;",
     "out->frag_one_minus_largest_over_free = 1.0 - F / L;"),
    ("stats_no_tail", "    if (tail > 0) {\n        out->hole_count += 1;",
     "    if (tail > arena_bytes) {\n        out->hole_count += 1;"),
    ("stats_cursor_start", "        cursor = offset[i] + size[i];\n    }\n    const uint64_t tail",
     "        cursor = offset[i];\n    }\n    const uint64_t tail"),
    ("window_hole_cursor_start", "        cursor = offset[i] + size[i];\n    }\n    if (arena_bytes > cursor)",
     "        cursor = offset[i];\n    }\n    if (arena_bytes > cursor)"),
    ("stats_counts_every_gap", "        if (gap > 0) {\n            out->hole_count += 1;",
     "        if (gap >= 0) {\n            out->hole_count += 1;"),
    ("stats_min_not_max", "            if (gap > out->largest_hole) out->largest_hole = gap;",
     "            if (gap < out->largest_hole) out->largest_hole = gap;"),
    ("stats_moved_inverted", "        if (offset[i] != new_off) {", "        if (offset[i] == new_off) {"),
    ("stats_zero_free_rule", "    if (out->free_bytes == 0) {", "    if (out->free_bytes == 1) {"),
    ("remap_one_past_end", "if (live[i] && h - offset[i] < size[i])", "if (live[i] && h - offset[i] <= size[i])"),
    ("remap_ignores_live", "if (live[i] && h - offset[i] < size[i])", "if (h - offset[i] < size[i])"),
    ("remap_drops_inner_offset", "result = new_off[i] + (h - offset[i]);", "result = new_off[i];"),
    ("remap_lower_bound", "std::upper_bound(offset, offset + n, h)", "std::lower_bound(offset, offset + n, h)"),
    ("validate_16_byte", "offset[i] % 32 != 0 || size[i] % 32 != 0", "offset[i] % 16 != 0 || size[i] % 16 != 0"),
    ("validate_touching_overlap", "offset[i - 1] + size[i - 1] > offset[i]", "offset[i - 1] + size[i - 1] >= offset[i]"),
    ("validate_exact_fit_rejected", "size[i] > arena_bytes - offset[i]", "size[i] >= arena_bytes - offset[i]"),
    ("validate_order_swapped", "        if (size[i] == 0)\n            r = ORACLE_REASON_ZERO_SIZE;\n        else if (offset[i] % 32 != 0 || size[i] % 32 != 0)\n            r = ORACLE_REASON_MISALIGNED;",
     "        if (offset[i] % 32 != 0 || size[i] % 32 != 0)\n            r = ORACLE_REASON_MISALIGNED;\n        else if (size[i] == 0)\n            r = ORACLE_REASON_ZERO_SIZE;"),
    ("source_map_block_start", "emit(a, offset[i] + (a - dst), b - a)", "emit(a, offset[i], b - a)"),
    ("pinned_segment_base_drops_size",
     "            new_offset[i] = offset[i];\n            running = offset[i] + size[i];",
     "            new_offset[i] = offset[i];\n            running = offset[i];"),
    ("pinned_blocks_move", "        if (is_pinned(pinned, i)) {\n            dst = offset[i] + size[i];\n            continue;\n        }\n        if (!live[i]) continue;\n        if (dst != offset[i])",
     "        if (!live[i]) continue;\n        if (dst != offset[i])"),
    ("pinned_free_accepted", "(pinned[i] == 1 && live[i] == 0)", "(pinned[i] == 3 && live[i] == 0)"),
    ("pinned_moved_counted", "        if (is_pinned(pinned, i)) {\n            new_off = offset[i] + size[i];\n        } else {",
     "        if (false) {\n        } else {"),
    ("window_not_shortest", "while (first < last && free_sum - holes[first].len >= request)",
     "while (first < last && free_sum - holes[first].len > request)"),
    ("window_exact_fit_rejected", "        if (free_sum < request) continue;", "        if (free_sum <= request) continue;"),
    ("window_highest_on_tie", "(live_sum == out->moved_bytes && begin < out->begin)",
     "(live_sum == out->moved_bytes && begin > out->begin)"),
    ("window_crosses_pinned", "            if (holes[last - 1].pinned_after) {  // start again past the barrier",
     "            if (false) {"),
    ("window_cost_not_dropped", "            live_sum -= holes[first].live_after;\n", ""),
    ("first_fit_exact_rejected", "        if (offset[i] - cursor >= need) {", "        if (offset[i] - cursor > need) {"),
    ("first_fit_no_rounding", "    const uint64_t need = (request + 31) / 32 * 32;", "    const uint64_t need = request;"),
    ("first_fit_round_16", "    const uint64_t need = (request + 31) / 32 * 32;",
     "    const uint64_t need = (request + 15) / 16 * 16;"),
    ("first_fit_hole_end", "            *offset_out = cursor;\n            return ORACLE_OK;",
     "            *offset_out = offset[i] - need;\n            return ORACLE_OK;"),
    ("first_fit_tail_ignored", "    if (arena_bytes - cursor >= need) *offset_out = cursor;", ""),
    ("monitor_critical_inclusive", "    if (usage > critical_ratio)", "    if (usage >= critical_ratio)"),
    ("monitor_warning_inclusive", "    else if (usage > warning_ratio)", "    else if (usage >= warning_ratio)"),
    ("monitor_levels_swapped", "        out->level = ORACLE_LEVEL_CRITICAL;\n    else if (usage > warning_ratio)\n        out->level = ORACLE_LEVEL_WARNING;",
     "        out->level = ORACLE_LEVEL_WARNING;\n    else if (usage > warning_ratio)\n        out->level = ORACLE_LEVEL_CRITICAL;"),
    ("monitor_no_rounding", "        const uint64_t need = huge ? UINT64_MAX : (next_request + 31) / 32 * 32;",
     "        const uint64_t need = huge ? UINT64_MAX : next_request;"),
    ("monitor_capacity_inverted", "            out->action = (!huge && need <= free_bytes) ? ORACLE_ACTION_TARGETED",
     "            out->action = (!huge && need > free_bytes) ? ORACLE_ACTION_TARGETED"),
    ("monitor_time_from_used", "                               ? (double)free_bytes / growth_bytes_per_s",
     "                               ? (double)live_bytes / growth_bytes_per_s"),
    ("monitor_threshold_inclusive", "out->frag_free_over_largest_minus_1 > frag_threshold)",
     "out->frag_free_over_largest_minus_1 >= frag_threshold)"),
    ("monitor_request_ignored", "    if (next_request > 0) {", "    if (next_request > UINT64_MAX) {"),
    ("window_tail_ignored", "    if (arena_bytes > cursor) holes.push_back(Hole{cursor, arena_bytes - cursor, 0, false});",
     ""),
]


def _battery():
    """Run the pins; return True if all hold."""
    try:
        for case in T._golden():
            T.test_golden_hand_worked(case, None)
        rng = np.random.default_rng(99)
        for k in range(60):
            heap = W.tiny_heap(rng, int(rng.integers(0, 25)), sizes=(32, 64, 96, 160, 4096),
                               gap_p=[0.0, 0.3, 0.8][k % 3], live_p=[0.3, 0.6, 1.0][k % 3],
                               pinned_p=[0.0, 0.3][k % 2])
            T._check_against_bruteforce(heap)
            T._check_source_map_windows(heap, rng, 4)
        for table, S, idx, reason in [
                ([(0, 0, 1)], 64, 0, 1), ([(16, 32, 1)], 64, 0, 2), ([(0, 48, 1)], 64, 0, 2),
                ([(0, 32, 2)], 64, 0, 3), ([(0, 32, 1), (32, 64, 1)], 64, 1, 4),
                ([(0, 64, 1), (32, 32, 0)], 128, 1, 5), ([(16, 0, 1)], 64, 0, 1)]:
            T.test_validation_reasons(table, S, idx, reason, None)
        T.test_validation_reasons_pinned([(0, 32, 0)], [1], 64, 0, 7, None)
        # a valid table that fills the arena exactly and touches neighbours
        t = np.array([(0, 32, 1), (32, 32, 1)], dtype=np.uint64)
        assert oracle.validate(t[:, 0], t[:, 1], t[:, 2].astype(np.uint8), 64)[0] == oracle.OK
        T.test_empty_and_degenerate(None)
        for case in TT.golden_cases():
            TT.check_golden(case)
        for k in range(40):
            heap = W.tiny_heap(rng, int(rng.integers(0, 16)), sizes=(32, 64, 96, 160, 1024),
                               gap_p=[0.0, 0.3, 0.8][k % 3], live_p=[0.3, 0.6, 1.0][k % 3],
                               pinned_p=[0.0, 0.3][k % 2])
            TT.check_against_bruteforce(heap, rng)
            FF.check_against_bruteforce(heap, rng)
            FF.check_proof(heap, rng)
        FF.check_golden()
        for case in MO.golden_cases():
            MO.check_case(case, oracle.monitor)
    except AssertionError:
        return False
    return True


def test_unmodified_oracle_passes_battery():
    assert _battery()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), d)
        cpp = os.path.join(d, "oracle.cpp")
        open(cpp, "w").write(text.replace(old, new))
        so = os.path.join(d, "liboracle_mut.so")
        subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-w", "-o", so, cpp],
                       check=True)
        prev = oracle.swap_library(so)
        try:
            assert not _battery(), f"the pins did not catch mutant {name}"
        finally:
            oracle.restore_library(prev)
    finally:
        shutil.rmtree(d, ignore_errors=True)

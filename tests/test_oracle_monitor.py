"""Pins for the oracle's layout monitor (oracle_monitor): decisions and
figures worked by hand from the pages (tests/golden/monitor_hand_worked.json)
and properties of the definition over random inputs."""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_cases():
    with open(os.path.join(HERE, "golden", "monitor_hand_worked.json")) as f:
        return json.load(f)["cases"]


def check_case(c, run):
    """run(arena, live, largest, warning, critical, tau, request, growth)
    -> Monitor-like with level, action, usage_ratio, r1, seconds_to_full."""
    m = run(c["arena_bytes"], c["live_bytes"], c["largest_hole"], 0.85, 0.95,
            float(c["frag_threshold"]), c["next_request"], float(c["growth"]))
    e = c["expect"]
    assert oracle.LEVELS[m.level] == e["level"], c["name"]
    assert oracle.ACTIONS[m.action] == e["action"], c["name"]
    un, ud = e["usage_num_den"]
    assert m.usage_ratio == un / ud, c["name"]
    if e["r1_num_den"] is None:
        assert m.frag_free_over_largest_minus_1 == 0.0
    else:
        rn, rd = e["r1_num_den"]
        assert m.frag_free_over_largest_minus_1 == rn / rd - 1.0, c["name"]
    if e["seconds_to_full"] == "inf":
        assert math.isinf(m.seconds_to_full) and m.seconds_to_full > 0
    else:
        assert m.seconds_to_full == e["seconds_to_full"], c["name"]


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_golden_monitor(case, oracle_lib):
    check_case(case, oracle.monitor)


def check_properties(rng, n=3000):
    for _ in range(n):
        S = int(rng.integers(1, 1 << 40))
        live = int(rng.integers(0, S + 1))
        F = S - live
        largest = int(rng.integers(1, F + 1)) if F else 0
        req = int(rng.choice([0, int(rng.integers(1, 2 * S + 64))]))
        tau = float(rng.choice([0.0, rng.uniform(0, 10)]))
        g = float(rng.choice([0.0, -1.0, rng.uniform(1, 1e9)]))
        m = oracle.monitor(S, live, largest, 0.85, 0.95, tau, req, g)
        need = -(-req // 32) * 32
        if req and need > largest:
            assert oracle.ACTIONS[m.action] == ("targeted" if need <= F else "no_room")
        elif tau > 0 and F and F / largest - 1 > tau:
            assert oracle.ACTIONS[m.action] == "full"
        else:
            assert oracle.ACTIONS[m.action] == "none"
        u = live / S
        assert m.level == (2 if u > 0.95 else 1 if u > 0.85 else 0)
        assert (m.seconds_to_full == F / g) if g > 0 else math.isinf(m.seconds_to_full)


def test_properties(oracle_lib):
    check_properties(np.random.default_rng(17))

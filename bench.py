#!/usr/bin/env python3
"""Benchmark: in-place compaction of the 80 GiB training arena on one MI355X.

One step = the whole hot path on one fragmented arena:
  plan   (validate, live-size scan, hole statistics, mover tile table)
  move   (the in-place mover)
  remap  (4,000,000 handles)
  commit + statistics of the packed table (one top hole, ratios 0).
Before every step the arena is refilled to its pristine fragmented content on
the GPU; the refill sits outside the timed events (inputs resident in HBM when
a step starts).  It is one device copy from a pristine snapshot kept in HBM:
regenerating the payload with torch ops takes ~1,500 launches, after which
the runtime's next calls ran 0.3-0.5 ms late on the host, a cost that
belongs to the refill and not to the step (--regen-refill keeps that way).

The step is timed twice, with HIP events on the stream the library launches
on: through defrag_compact (the whole operator in one C-ABI call, which
queues the move behind the plan without waiting for the host: the headline
value) and through the separate calls, one event between each phase (the
per-phase times; the mover launch has its own event pair, which gives the
roofline figure).

Prints one JSON line.  --gpus N > 1 is refused: each GPU compacts its own arena, so
the benchmark runs on one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak (8 TB/s)
METRIC = "compaction GB/s moved (read+write) & % HBM peak; handles remapped/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "move_training80g_traffic.json")


def _mover_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("move.hip", "internal.h"):
        with open(os.path.join(ROOT, "arena_compaction_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(moved_bytes: int):
    """Measured HBM bytes per mover launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy of known size), if taken on the current mover
    source for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("mover_source_hash") != _mover_source_hash() or t.get("moved_bytes") != moved_bytes:
        return None
    return t.get("hbm_bytes_per_launch")


def _host_description() -> str:
    """CPU model, logical CPUs and RAM of the host the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    mem = 0
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    mem = int(line.split()[1]) * 1024
                    break
    except OSError:
        pass
    return f"{model}; {os.cpu_count()} logical CPUs; {mem / 2**30:.0f} GiB RAM"


def cpu_baseline(heap, reps: int = 3):
    """The oracle as it stands, single-threaded, on the whole heap the GPU
    compacts (every entry, every byte of the arena, every handle): validate +
    new offsets + statistics, the ordered memmove, and the remap, each timed
    on its own; median of ``reps`` runs, the arena restored to its pristine
    payload before each run (untimed; the generator fills it on all cores).
    Needs the arena's size in host memory."""
    import numpy as np
    import torch
    import oracle
    import workloads as W

    S = heap.arena_bytes
    off, size, live, hs = heap.offset, heap.size, heap.live, heap.handles
    arena = np.empty(S, dtype=np.uint8)
    at = torch.from_numpy(arena)
    phases = {"plan_stats": [], "memmove": [], "remap": []}
    moved = None
    for r in range(reps):
        W.fill_payload(at, 0, heap.payload_mode, heap.payload_seed)
        t0 = time.perf_counter()
        rc = oracle.validate(off, size, live, S, pinned=heap.pinned)[0]
        oracle.new_offsets(off, size, live, heap.pinned)
        st = oracle.stats(off, size, live, S, pinned=heap.pinned)
        t1 = time.perf_counter()
        oracle.compact(arena, off, size, live, heap.pinned)
        t2 = time.perf_counter()
        oracle.remap(off, size, live, hs, pinned=heap.pinned)
        t3 = time.perf_counter()
        assert rc == oracle.OK
        moved = st.moved_bytes
        phases["plan_stats"].append(t1 - t0)
        phases["memmove"].append(t2 - t1)
        phases["remap"].append(t3 - t2)
        print(f"# cpu baseline run {r}: plan+stats {t1 - t0:.3f} s, memmove {t2 - t1:.3f} s, "
              f"remap {t3 - t2:.3f} s", file=sys.stderr, flush=True)
    del at, arena
    med = {k: float(np.median(v)) for k, v in phases.items()}
    total = sum(med.values())
    return {
        "value": round(2 * moved / total / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "host": _host_description(),
        "sample": (f"the whole {heap.name} heap ({S} B arena, {heap.n} entries, {moved} B "
                   f"moved, {hs.shape[0]} handles): validate + new offsets + statistics, "
                   f"ordered memmove, remap; median of {reps} runs, arena restored untimed "
                   f"between runs"),
        "seconds_per_compaction": round(total, 3),
        "seconds": {k: round(v, 4) for k, v in med.items()},
        "memmove_GBps": round(2 * moved / med["memmove"] / 1e9, 3),
        "handles_per_s": round(hs.shape[0] / med["remap"], 1),
    }


def ablation_waves(args, heap, arena, off, size, live, pinned, ws, tuning) -> int:
    """Shift-sized waves against the tiled mover.  Correct in-place order
    without the mover's tile flags: blocks strictly ascending, and inside a
    block copies of at most its shift, so a copy never overlaps its own
    source and never overwrites a source not yet copied.  Each copy is one
    device-to-device copy kernel (torch), issued back to back on one stream."""
    import numpy as np
    import torch
    import arena_compaction_amd as ac
    import workloads as W
    S = heap.arena_bytes
    new = torch.empty(heap.n, dtype=torch.int64, device=arena.device)
    plan = ac.defrag_plan(off, size, live, S, ws, new, tuning=tuning, pinned=pinned)
    new_h = new.cpu().numpy().view(np.uint64)
    li = np.flatnonzero(heap.live)
    waves = []
    for i in li.tolist():
        o, n, d = int(heap.offset[i]), int(heap.size[i]), int(new_h[i])
        sh = o - d
        if sh == 0:
            continue
        for c in range(0, n, sh):
            ln = min(sh, n - c)
            waves.append((d + c, o + c, ln))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    # tiled mover
    ev[0].record()
    ac.defrag_move(arena, plan, ws)
    ev[1].record()
    assert ac.defrag_move_status(plan, ws) == ac.DEFRAG_OK
    tiled = arena.clone()
    # waves, on a fresh copy of the same input
    W.fill_payload(arena, 0, heap.payload_mode, heap.payload_seed)
    torch.cuda.synchronize()
    t0 = time.time()
    ev[2].record()
    for d, s0, ln in waves:
        arena[d:d + ln].copy_(arena[s0:s0 + ln])
    ev[3].record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    equal = bool(torch.equal(arena, tiled))
    moved = int(plan.stats.moved_bytes)
    t_tiled = ev[0].elapsed_time(ev[1])
    t_waves = ev[2].elapsed_time(ev[3])
    print(json.dumps({
        "ablation": "shift-sized waves (one copy per wave, blocks ascending) vs tiled mover",
        "workload": heap.describe(), "moved_bytes": moved, "waves": len(waves),
        "tiled_ms": round(t_tiled, 3), "tiled_GBps": round(2 * moved / t_tiled / 1e6, 1),
        "waves_ms": round(t_waves, 3), "waves_GBps": round(2 * moved / t_waves / 1e6, 1),
        "waves_host_wall_s": round(wall, 3),
        "tiled_speedup": round(t_waves / t_tiled, 2), "bytes_equal": equal}), flush=True)
    return 0 if equal else 1


def latency(args, heap, arena, off, size, live, pinned, ws, tuning, h_in, h_out, n_bad, new_off,
            c_off, c_size, c_live, c_pin) -> int:
    """Wall time per call, in microseconds, of the one-call path and its
    pieces: the C function called directly with its argument struct built
    once (the binding's marshalling timed apart), each call ending in its
    own read-back, so back-to-back calls do not overlap."""
    import ctypes
    import torch
    import arena_compaction_amd as ac
    S = heap.arena_bytes
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    reps = max(args.steps, 1) * 20
    out = {}

    def timeit(name, fn):
        for _ in range(max(args.warmup, 1) * 3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name] = round((time.perf_counter() - t0) / reps * 1e6, 1)

    full = dict(handles=h_in, h_out=h_out, n_invalid=n_bad, offset_out=c_off, size_out=c_size,
                live_out=c_live, pinned_out=c_pin)
    variants = {
        "one_call": (full, True),
        "one_call_no_post_check": (full, False),
        "plan_move_commit": (dict(offset_out=c_off, size_out=c_size, live_out=c_live,
                                  pinned_out=c_pin), False),
        "plan_move": ({}, False),
    }
    for name, (kw, after) in variants.items():
        a, keep = ac._compact_args(off, size, live, S, arena, ws, 0, new_off, kw.get("handles"),
                                   kw.get("h_out"), kw.get("n_invalid"), kw.get("offset_out"),
                                   kw.get("size_out"), kw.get("live_out"), kw.get("pinned_out"),
                                   tuning, pinned)
        plan, post = ac.defrag_plan_t(), ac.defrag_stats_t()

        def call(a=a, plan=plan, post=post, after=after):
            rc = ac.lib.defrag_compact(ctypes.byref(a), sp, ctypes.byref(plan),
                                       ctypes.byref(post) if after else None)
            if rc != ac.DEFRAG_OK:
                raise ac.DefragError(rc, "defrag_compact")
        timeit(name, call)
    timeit("binding_marshalling", lambda: ac._compact_args(
        off, size, live, S, arena, ws, 0, new_off, h_in, h_out, n_bad, c_off, c_size, c_live,
        c_pin, tuning, pinned))
    timeit("plan_via_binding", lambda: ac.defrag_plan(off, size, live, S, ws, new_off,
                                                      tuning=tuning, stream=stream, pinned=pinned))
    timeit("stats_via_binding", lambda: ac.defrag_stats(off, size, live, S, ws, stream=stream,
                                                        pinned=pinned))
    print(json.dumps({"workload": heap.name, "entries": heap.n, "live_blocks": int(heap.live.sum()),
                      "handles": int(heap.handles.size), "calls_per_figure": reps,
                      "us_per_call": out}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="training-80g",
                    help="one of mixed-64m, pairs-1g, training-80g (the headline), "
                         "training-80g-pinned, small-blocks-4g, overlap-64g")
    ap.add_argument("--tile", type=int, default=None, help="override the mover tile bytes")
    ap.add_argument("--wg-per-cu", type=int, default=None, help="override (0 = max occupancy)")
    ap.add_argument("--nontemporal", type=int, default=None, help="override (0..3)")
    ap.add_argument("--request", type=int, default=None,
                    help="bytes for the targeted-compaction leg (default: 4.2/80 of the arena "
                         "for the training-80g workloads -- the 910C page's 4.2 GB buffer -- "
                         "else off; "
                         "0 turns it off)")
    ap.add_argument("--ablation-waves", action="store_true",
                    help="instead of the benchmark: time the alternative the tiled mover "
                         "replaces -- every moved block copied in ascending order in waves of at "
                         "most its shift (one copy per wave, so no wave overlaps its own "
                         "source) -- against defrag_move on the same arena, and compare bytes")
    ap.add_argument("--regen-refill", action="store_true",
                    help="refill the arena before each step by regenerating the payload with "
                         "torch ops instead of copying a pristine snapshot")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3,
                    help="runs of the CPU oracle on the whole heap (median reported)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="GIB",
                    help="only run a plain device-to-device copy of GIB GiB (twice): the "
                         "reference kernel that scales the HBM byte counters")
    ap.add_argument("--calibrate-move", type=int, default=0, metavar="GIB",
                    help="only run the mover (twice) on one GIB GiB block that moves down by "
                         "GIB GiB: a plain copy of known size with the mover's own streaming "
                         "loads and stores and no dependency, to scale the byte counters of "
                         "its non-temporal accesses")
    ap.add_argument("--latency", action="store_true",
                    help="instead of the benchmark: the wall time of one defrag_compact call "
                         "through the C-ABI (arguments built once, the call's own final "
                         "read-back included), with and without each piece of the step, and of "
                         "defrag_plan and defrag_stats alone; the arena is not refilled "
                         "between calls (a repeated compaction moves the same bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; each GPU compacts "
                                   "its own arena independently, so there is no multi-GPU step",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import numpy as np
    import torch
    import arena_compaction_amd as ac
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        nb = args.calibrate_copy << 30
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(2):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nb, "copies": 2}), flush=True)
        return 0
    if args.calibrate_move:
        nb = args.calibrate_move << 30
        heap = W.table_from_lists(2 * nb, [(0, nb), (nb, nb)], [0, 1], [], name="calibrate")
        o_, s_, l_ = (torch.from_numpy(heap.offset.view(np.int64)).to(dev),
                      torch.from_numpy(heap.size.view(np.int64)).to(dev),
                      torch.from_numpy(heap.live).to(dev))
        a = torch.zeros(2 * nb, dtype=torch.uint8, device=dev)
        ws = ac.workspace(heap.n, 2 * nb, device=dev)
        for _ in range(2):
            p = ac.defrag_plan(o_, s_, l_, 2 * nb, ws)
            ac.defrag_move(a, p, ws)
            assert ac.defrag_move_status(p, ws) == ac.DEFRAG_OK
            rep = ac.defrag_move_report(p, ws)
            assert rep.late_tiles == 0
        print(json.dumps({"calibrate_move_bytes": nb, "moves": 2, "tiles": int(p.n_tiles)}),
              flush=True)
        return 0
    t_gen = time.time()
    heap = W.workload(args.workload)
    S = heap.arena_bytes
    off = torch.from_numpy(heap.offset.view(np.int64)).to(dev)
    size = torch.from_numpy(heap.size.view(np.int64)).to(dev)
    live = torch.from_numpy(heap.live).to(dev)
    pinned = None if heap.pinned is None else torch.from_numpy(heap.pinned).to(dev)
    h_in = torch.from_numpy(heap.handles.view(np.int64)).to(dev)
    h_out = torch.empty_like(h_in)
    n_bad = torch.zeros(1, dtype=torch.int64, device=dev)
    arena = torch.empty(S, dtype=torch.uint8, device=dev)
    tuning = None   # library defaults unless a knob is overridden
    if args.tile is not None or args.wg_per_cu is not None or args.nontemporal is not None:
        tuning = ac.defrag_tuning(args.tile or 0, 1 if args.wg_per_cu is None else args.wg_per_cu,
                                  1 if args.nontemporal is None else args.nontemporal, 0)
    ws = ac.workspace(heap.n, S, args.tile or 0, device=dev, max_pinned=heap.n_pinned)
    new_off = torch.empty(heap.n, dtype=torch.int64, device=dev)
    m = int(heap.live.sum())
    c_off = torch.empty(m, dtype=torch.int64, device=dev)
    c_size = torch.empty(m, dtype=torch.int64, device=dev)
    c_live = torch.empty(m, dtype=torch.uint8, device=dev)
    c_pin = torch.empty(m, dtype=torch.uint8, device=dev)
    W.fill_payload(arena, 0, heap.payload_mode, heap.payload_seed)
    torch.cuda.synchronize()
    print(f"# {heap.describe()} generated+filled in {time.time() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    if args.ablation_waves:
        return ablation_waves(args, heap, arena, off, size, live, pinned, ws, tuning)
    if args.latency:
        return latency(args, heap, arena, off, size, live, pinned, ws, tuning, h_in, h_out, n_bad,
                       new_off, c_off, c_size, c_live, c_pin)
    stream = torch.cuda.current_stream()
    refill_from = 0
    snap = {"from": None, "bytes": None}   # pristine bytes [from, S), when they fit

    def refill():
        # bytes below the first destination are never written: refill the rest
        a0 = (refill_from // 8) * 8
        if not args.regen_refill and snap["from"] != a0:
            snap["bytes"] = None
            snap["from"] = a0
            try:
                t = torch.empty(S - a0, dtype=torch.uint8, device=dev)
                W.fill_payload(t, a0, heap.payload_mode, heap.payload_seed)
                snap["bytes"] = t
            except torch.cuda.OutOfMemoryError:
                torch.cuda.empty_cache()
        if snap["bytes"] is not None:
            arena[a0:].copy_(snap["bytes"])
        else:
            W.fill_payload(arena[a0:], a0, heap.payload_mode, heap.payload_seed)

    def one_call(request=0):
        # the whole step through one C-ABI call (defrag_compact)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        plan, post = ac.defrag_compact(off, size, live, S, arena, ws, request, new_off, h_in,
                                       h_out, n_bad, c_off, c_size, c_live, c_pin, tuning=tuning,
                                       stream=stream, pinned=pinned)
        ev[1].record(stream)
        return plan, post, ev

    def one_step():
        # the same step through the separate calls, one event between each
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record(stream)
        plan = ac.defrag_plan(off, size, live, S, ws, new_off, tuning=tuning, stream=stream,
                              pinned=pinned)
        ev[1].record(stream)
        ac.defrag_move(arena, plan, ws, stream=stream)
        ev[2].record(stream)
        ac.defrag_remap(plan, ws, h_in, h_out, n_bad, stream=stream)
        ev[3].record(stream)
        ac.defrag_commit(plan, ws, c_off, c_size, c_live, stream=stream, pinned_out=c_pin)
        post = ac.defrag_stats(c_off, c_size, c_live, S, ws, stream=stream, pinned=c_pin)
        ev[4].record(stream)
        return plan, post, ev

    for w in range(args.warmup):
        refill()
        torch.cuda.synchronize()
        plan, post, ev = one_step()
        assert ac.defrag_move_status(plan, ws) == ac.DEFRAG_OK
        refill_from = int(plan.move_begin)
        print(f"# warmup {w} done", file=sys.stderr, flush=True)

    for w in range(args.warmup):
        refill()
        torch.cuda.synchronize()
        one_call()
    times = {"step": [], "one_call": [], "plan": [], "move": [], "remap": [], "post": []}
    torch.cuda.synchronize()
    t_wall0 = time.time()
    moved = None
    for k in range(args.steps):   # the timed steps, one event between each phase
        refill()
        torch.cuda.synchronize()
        plan, post, ev = one_step()
        torch.cuda.synchronize()
        st = ac.defrag_move_status(plan, ws)
        assert st == ac.DEFRAG_OK, st
        rep = ac.defrag_move_report(plan, ws)
        if heap.pinned is None:   # one top hole afterwards
            assert post.hole_count == (1 if post.free_bytes else 0)
            assert post.frag_free_over_largest_minus_1 == 0.0
        assert int(n_bad.item()) == 0
        moved = int(plan.stats.moved_bytes)
        times["step"].append(ev[0].elapsed_time(ev[4]))
        times["plan"].append(ev[0].elapsed_time(ev[1]))
        times["move"].append(ev[1].elapsed_time(ev[2]))
        times["remap"].append(ev[2].elapsed_time(ev[3]))
        times["post"].append(ev[3].elapsed_time(ev[4]))
        print(f"# step {k}: step {times['step'][-1]:.3f} ms, move {times['move'][-1]:.3f} ms",
              file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.time() - t_wall0
    for k in range(args.steps):   # the same steps through defrag_compact, for comparison
        refill()
        torch.cuda.synchronize()
        plan, post, ev = one_call()
        torch.cuda.synchronize()
        assert int(n_bad.item()) == 0 and int(plan.stats.moved_bytes) == moved
        times["one_call"].append(ev[0].elapsed_time(ev[1]))
    torch.cuda.synchronize()
    full_plan = plan

    # Targeted leg: the smallest move that frees one hole of the request.
    request = args.request
    if request is None:
        request = S * 42 // 800 if args.workload.startswith("training-80g") else 0
    targeted = None
    if request:
        tt = {"step": [], "one_call": [], "plan": [], "move": [], "remap": [], "post": []}
        for k in range(args.warmup + args.steps):
            refill()
            torch.cuda.synchronize()
            tp, tpost, ev = one_call(request)
            torch.cuda.synchronize()
            assert tpost.largest_hole >= request and int(n_bad.item()) == 0
            if k >= args.warmup:
                tt["one_call"].append(ev[0].elapsed_time(ev[1]))
        for k in range(args.warmup + args.steps):
            refill()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record(stream)
            tp = ac.defrag_plan_targeted(off, size, live, S, request, ws, new_off,
                                         tuning=tuning, stream=stream, pinned=pinned)
            ev[1].record(stream)
            ac.defrag_move(arena, tp, ws, stream=stream)
            ev[2].record(stream)
            ac.defrag_remap(tp, ws, h_in, h_out, n_bad, stream=stream)
            ev[3].record(stream)
            ac.defrag_commit(tp, ws, c_off, c_size, c_live, stream=stream, pinned_out=c_pin)
            tpost = ac.defrag_stats(c_off, c_size, c_live, S, ws, stream=stream, pinned=c_pin)
            ev[4].record(stream)
            torch.cuda.synchronize()
            assert ac.defrag_move_status(tp, ws) == ac.DEFRAG_OK
            assert tpost.largest_hole >= request and int(n_bad.item()) == 0
            if k >= args.warmup:
                for key, (a, b) in (("step", (0, 4)), ("plan", (0, 1)), ("move", (1, 2)),
                                    ("remap", (2, 3)), ("post", (3, 4))):
                    tt[key].append(ev[a].elapsed_time(ev[b]))
        tmean = {k: float(np.mean(v)) for k, v in tt.items()}
        tmoved = int(tp.stats.moved_bytes)
        # the allocation the page's request failed to get, before and after,
        # and what the layout monitor says about each state
        ff_before, st_before = ac.defrag_first_fit(off, size, live, S, request, ws, pinned=pinned)
        ff_after, _ = ac.defrag_first_fit(c_off, c_size, c_live, S, request, ws, pinned=c_pin)
        ff_ms = []   # first fit on the fragmented table: one statistics pass, one read-back
        for k in range(args.warmup + args.steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            ac.defrag_first_fit(off, size, live, S, request, ws, stream=stream, pinned=pinned)
            ev[1].record(stream)
            torch.cuda.synchronize()
            if k >= args.warmup:
                ff_ms.append(ev[0].elapsed_time(ev[1]))
        mon_before = ac.defrag_monitor(st_before, next_request=request)
        mon_after = ac.defrag_monitor(tpost, next_request=request)
        targeted = {
            "request_bytes": request,
            "window": [int(tp.window_begin), int(tp.window_end)],
            "hole_bytes": int(tp.window_hole),
            "moved_bytes": tmoved,
            "moved_vs_full": round(tmoved / moved, 4) if moved else None,
            "ms": {k: round(v, 4) for k, v in tmean.items()},
            "step_vs_full": round(tmean["step"] / float(np.mean(times["step"])), 4),
            "move_GBps": round(2 * tmoved / (tmean["move"] * 1e-3) / 1e9, 2) if tmoved else None,
            "after_largest_hole": int(tpost.largest_hole),
            "first_fit_before": ff_before,
            "first_fit_after": ff_after,
            "first_fit_ms": round(float(np.mean(ff_ms)), 4),
            "monitor_before": {"level": ac.LEVELS[mon_before.level],
                               "action": ac.ACTIONS[mon_before.action]},
            "monitor_after": {"level": ac.LEVELS[mon_after.level],
                              "action": ac.ACTIONS[mon_after.action]},
        }
        print(f"# targeted: request {request} moved {tmoved} step {tmean['step']:.3f} ms",
              file=sys.stderr, flush=True)

    mean = {k: float(np.mean(v)) for k, v in times.items()}
    ms_step = mean["one_call"]   # the whole operator through one call
    value = 2 * moved / (ms_step * 1e-3) / 1e9
    value_separate = 2 * moved / (mean["step"] * 1e-3) / 1e9
    move_gbps = 2 * moved / (mean["move"] * 1e-3) / 1e9
    handles_per_s = heap.handles.shape[0] / (mean["remap"] * 1e-3)
    traffic = _traffic(moved)
    s0 = full_plan.stats
    plan = full_plan
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {W.SUMMARY[args.workload]}",
            "arena_bytes": S, "entries": heap.n, "live_blocks": m,
            "handles": int(heap.handles.shape[0]), "moved_bytes": moved,
            "pinned_blocks": heap.n_pinned,
            "tile_bytes": int(plan.tuning.tile_bytes), "seed": heap.seed,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "step_api": "defrag_compact (one call: plan, move, remap, commit, post-check)",
        "value_separate_calls": round(value_separate, 2),
        "move_only_GBps": round(move_gbps, 2),
        "move_pct_hbm_peak": round(100 * move_gbps / HBM_PEAK_GBPS, 2),
        "handles_per_s": round(handles_per_s, 1),
        "ms": {k: round(v, 4) for k, v in mean.items()},
        "mover_waits": {"tiles": int(rep.tiles), "late_tiles": int(rep.late_tiles),
                        "waited_tiles": int(rep.waited_tiles), "polls": int(rep.polls)},
        "min_move_ms": round(float(np.min(times["move"])), 4),
        "median_move_ms": round(float(np.median(times["move"])), 4),
        "max_move_GBps": round(2 * moved / (float(np.min(times["move"])) * 1e-3) / 1e9, 2),
        "wall_s_incl_refill": round(wall, 3),
        "refill": ("device copy of a pristine snapshot" if snap["bytes"] is not None
                   else "payload regenerated with torch ops"),
        "before": {"free_bytes": int(s0.free_bytes), "largest_hole": int(s0.largest_hole),
                   "hole_count": int(s0.hole_count),
                   "frag_free_over_largest_minus_1": s0.frag_free_over_largest_minus_1,
                   "frag_one_minus_largest_over_free": s0.frag_one_minus_largest_over_free},
        "after": {"largest_hole": int(post.largest_hole), "hole_count": int(post.hole_count),
                  "frag_free_over_largest_minus_1": post.frag_free_over_largest_minus_1},
        "targeted": targeted,
        "context_910c_page": {
            "note": "the pages' own figures, another machine and workload: context, not a target",
            "seconds_per_compaction": 1.2, "frag_free_over_largest_minus_1": [4.7, 0.8],
            "largest_hole_GB": [3, 12], "hbm_GB": 96, "hbm_TBps": 1.8},
        "target": {"frac_of_hbm_peak_on_moved_bytes": 0.70,
                   "met_by_mover": move_gbps / HBM_PEAK_GBPS >= 0.70},
        "roofline": {
            "bound": "hbm",
            "kernel": "k_move (defrag_move)",
            "achieved": round(move_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(move_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": 2 * moved,
        },
    }
    if not args.no_cpu_baseline and args.workload == "training-80g":
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(heap, args.cpu_reps)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and answers the calls that need no GPU (sizes, error text, and
argument errors caught on the host before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arena_compaction.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(defrag_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    fns = _declared_functions()
    for f in ("defrag_stats", "defrag_first_fit", "defrag_plan", "defrag_plan_targeted",
              "defrag_compact", "defrag_move", "defrag_remap",
              "defrag_workspace_bytes", "defrag_strerror", "defrag_commit",
              "defrag_move_status", "defrag_move_report", "defrag_plan_tiles",
              "defrag_compact_static"):
        assert f in fns, f


def test_library_exports_every_declared_symbol():
    import arena_compaction_amd as ac
    lib = ctypes.CDLL(ac.LIB_PATH)
    for f in _declared_functions():
        assert hasattr(lib, f), f"{f} declared in the header but not exported"
    assert set(_declared_functions()) == set(ac.EXPORTS)


def test_strerror_and_codes():
    import arena_compaction_amd as ac
    assert ac.defrag_strerror(0) == "ok"
    for c in (-1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert ac.defrag_strerror(c) not in ("ok", "unknown error")
    assert ac.defrag_strerror(-99) == "unknown error"


def test_workspace_bytes():
    import arena_compaction_amd as ac
    a = ac.defrag_workspace_bytes(0, 0)
    assert a > 0 and a % 256 == 0
    b = ac.defrag_workspace_bytes(4096, 64 << 20)
    c = ac.defrag_workspace_bytes(8192, 64 << 20)
    d = ac.defrag_workspace_bytes(4096, 64 << 20, 256)
    assert a < b < c and b < d
    # 80 GiB arena, 200k entries, default tiles: about 0.1% of the arena
    big = ac.defrag_workspace_bytes(200_247, 80 << 30)
    assert big < 128 << 20
    # room for pinned entries grows it only by the tiles they may add
    pinned = ac.defrag_workspace_bytes(200_247, 80 << 30, 0, 40)
    assert big < pinned < big + 40 * 2 * 64
    assert ac.defrag_workspace_bytes(10, 4096, 0, 11) == 0   # more pinned than entries
    for bad_tile in (100, 128, 3000, 524288):
        assert ac.defrag_workspace_bytes(16, 4096, bad_tile) == 0
    # more mover tiles than 32-bit tile indices (with room for the grid) allow
    assert ac.defrag_workspace_bytes(16, 1 << 44, 256) == 0
    assert ac.defrag_workspace_bytes(16, 0xFFFEFFF0 * 256, 256) > 0


def test_host_side_argument_errors_need_no_gpu():
    import arena_compaction_amd as ac
    L = ac.lib
    plan = ac.defrag_plan_t()
    # a zeroed plan is refused before any HIP call
    assert L.defrag_move(None, 0, ctypes.byref(plan), None, 0, None) == ac.DEFRAG_ENOPLAN
    assert L.defrag_remap(ctypes.byref(plan), None, 0, None, None, 0, None, None) == ac.DEFRAG_ENOPLAN
    assert L.defrag_commit(ctypes.byref(plan), None, 0, None, None, None, None, None) == ac.DEFRAG_ENOPLAN
    assert L.defrag_move_status(ctypes.byref(plan), None, None) == ac.DEFRAG_ENOPLAN
    assert L.defrag_plan_tiles(ctypes.byref(plan), None, 0, None, 0, None) == ac.DEFRAG_ENOPLAN
    rep = ac.defrag_move_report_t()
    assert L.defrag_move_report(ctypes.byref(plan), None, None, ctypes.byref(rep)) == ac.DEFRAG_ENOPLAN
    assert L.defrag_move_report(ctypes.byref(plan), None, None, None) == ac.DEFRAG_EINVAL
    # missing table / output pointers
    st = ac.defrag_stats_t()
    assert L.defrag_stats(None, 0, None, 0, None, ctypes.byref(st)) == ac.DEFRAG_EINVAL
    assert st.invalid_reason == 6
    assert L.defrag_stats(None, 0, None, 0, None, None) == ac.DEFRAG_EINVAL
    assert L.defrag_plan(None, 0, None, None, 0, None, None, None) == ac.DEFRAG_EINVAL
    t = ac.defrag_table(None, None, None, 5)   # n > 0 with NULL arrays
    assert L.defrag_plan(ctypes.byref(t), 4096, None, None, 0, None, None,
                         ctypes.byref(plan)) == ac.DEFRAG_EINVAL
    t = ac.defrag_table(None, None, None, 0)
    # no workspace
    assert L.defrag_plan(ctypes.byref(t), 4096, None, None, 0, None, None,
                         ctypes.byref(plan)) == ac.DEFRAG_EWORKSPACE
    # misaligned workspace pointer (never dereferenced: refused on the host)
    assert L.defrag_stats(ctypes.byref(t), 4096, ctypes.c_void_p(0x1008), 1 << 20, None,
                          ctypes.byref(st)) == ac.DEFRAG_EWORKSPACE
    # targeted plan: a zero request and a missing plan are refused on the host
    assert L.defrag_plan_targeted(ctypes.byref(t), 4096, 0, None, ctypes.c_void_p(0x1000),
                                  1 << 20, None, None, ctypes.byref(plan)) == ac.DEFRAG_EINVAL
    assert plan.stats.invalid_reason == 6
    assert L.defrag_plan_targeted(ctypes.byref(t), 4096, 64, None, ctypes.c_void_p(0x1000),
                                  1 << 20, None, None, None) == ac.DEFRAG_EINVAL
    assert ac.defrag_strerror(ac.DEFRAG_ENOFIT) not in ("ok", "unknown error")
    # first fit: missing output, zero request and a request that rounds past 2^64
    off_out = ctypes.c_uint64(7)
    assert L.defrag_first_fit(ctypes.byref(t), 4096, 64, ctypes.c_void_p(0x1000), 1 << 20, None,
                              None, None) == ac.DEFRAG_EINVAL
    for bad_request in (0, (1 << 64) - 31):
        assert L.defrag_first_fit(ctypes.byref(t), 4096, bad_request, ctypes.c_void_p(0x1000),
                                  1 << 20, None, ctypes.byref(off_out),
                                  ctypes.byref(st)) == ac.DEFRAG_EINVAL
        assert off_out.value == (1 << 64) - 1 and st.invalid_reason == 6
    # one-call compaction: missing arguments are refused on the host
    assert L.defrag_compact(None, None, ctypes.byref(plan), None) == ac.DEFRAG_EINVAL
    assert plan.stats.invalid_reason == 6
    args = ac.defrag_compact_args()
    args.n_handles = 5   # handles announced, no pointers
    assert L.defrag_compact(ctypes.byref(args), None, ctypes.byref(plan), None) == ac.DEFRAG_EINVAL
    args = ac.defrag_compact_args()   # no table: refused by the plan, on the host
    assert L.defrag_compact(ctypes.byref(args), None, ctypes.byref(plan),
                            ctypes.byref(st)) == ac.DEFRAG_EINVAL
    assert L.defrag_compact(ctypes.byref(args), None, None, None) == ac.DEFRAG_EINVAL
    # bad tile size, too many sleeps for the wait-path knob
    for tu in (ac.defrag_tuning(100, 0, 0, 0), ac.defrag_tuning(0, 1, 1, 0, 1, 4097, 0, 0)):
        assert L.defrag_plan(ctypes.byref(t), 4096, ctypes.byref(tu), ctypes.c_void_p(0x1000),
                             1 << 20, None, None, ctypes.byref(plan)) == ac.DEFRAG_EINVAL


def test_binding_refuses_bad_buffers_before_any_call():
    """The binding checks what it can know -- device, layout, dtype and the
    lengths the kernels will touch -- and raises before the library is
    called (a CPU tensor or a short buffer would be read or written out of
    bounds on the GPU)."""
    import torch
    import arena_compaction_amd as ac
    with pytest.raises(ValueError):
        ac._ptr(torch.zeros(4, dtype=torch.int64))          # host memory
    with pytest.raises(ValueError):
        ac._need(torch.zeros(4, dtype=torch.int32), torch.int64, 0, "x")
    with pytest.raises(ValueError):
        ac._need(torch.zeros(3, dtype=torch.int64), torch.int64, 4, "x")
    ac._need(None, torch.int64, 4, "x")
    ac._need(torch.zeros(4, dtype=torch.int64), torch.int64, 4, "x")
    plan = ac.defrag_plan_t()
    plan.live_blocks = 10
    ws = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="offset_out"):
        ac.defrag_commit(plan, ws, torch.zeros(9, dtype=torch.int64))
    with pytest.raises(ValueError, match="pinned_out"):
        ac.defrag_commit(plan, ws, None, None, None, pinned_out=torch.zeros(10, dtype=torch.int64))
    h = torch.zeros(8, dtype=torch.int64)
    with pytest.raises(ValueError, match="h_out"):
        ac.defrag_remap(plan, ws, h, torch.zeros(7, dtype=torch.int64))
    with pytest.raises(ValueError, match="h_in"):
        ac.defrag_remap(plan, ws, h.int())
    with pytest.raises(ValueError, match="n_invalid"):
        ac.defrag_remap(plan, ws, h, None, torch.zeros(0, dtype=torch.int64))
    with pytest.raises(ValueError, match="new_offset"):
        ac.defrag_plan(h, h, None, 4096, ws, torch.zeros(7, dtype=torch.int64))
    with pytest.raises(ValueError, match="live"):
        ac.defrag_stats(h, h, torch.zeros(7, dtype=torch.uint8), 4096, ws)
    with pytest.raises(ValueError, match="arena"):
        ac.defrag_move(torch.zeros(4, dtype=torch.int64), plan, ws)


def test_oracle_is_not_linked_into_the_product():
    """The product library and binding never reference the oracle."""
    pkg = os.path.join(ROOT, "arena_compaction_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"


def test_build_is_quiet_and_device_code_has_no_packed_fp32():
    """Every source compiles under -Wall -Wextra with nothing printed (the
    build drops only the host pass's note that it does not know the
    device-only feature), and the gfx950 code of each kernel file holds no
    packed-FP32 arithmetic."""
    import subprocess
    import sys
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_acb", os.path.join(ROOT, "arena_compaction_amd", "build.py"))
    acb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(acb)
    import tempfile
    csrc = os.path.join(ROOT, "arena_compaction_amd", "csrc")
    with tempfile.TemporaryDirectory() as tmp:   # the library's own build line
        p = subprocess.run([acb.hipcc()] + acb.HIPCC_FLAGS +
                           [os.path.join(csrc, s) for s in acb.SOURCES] +
                           ["-o", os.path.join(tmp, "lib.so")],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    shown = [ln for ln in p.stdout.splitlines() if ln.strip() != acb.HOST_FEATURE_NOTE]
    assert p.returncode == 0 and not shown, shown
    flags = [f for f in acb.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    for src in [s for s in acb.SOURCES if s.endswith(".hip")]:
        p = subprocess.run([acb.hipcc()] + flags + ["--cuda-device-only", "-S", "-o", "-",
                                                    os.path.join(csrc, src)],
                           stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        assert p.returncode == 0, p.stderr[-2000:]
        asm = p.stdout
        assert "gfx950" in asm, src
        if "__global__" in open(os.path.join(csrc, src)).read():
            assert ".amdhsa_kernel" in asm, src
        for op in ("v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"):
            assert op not in asm, f"{src}: {op} in the device code"
    sys.stdout.flush()


def test_binding_structs_match_the_header():
    """sizeof and field offsets of every struct the binding mirrors, as the C
    compiler lays them out from the header."""
    import ctypes
    import subprocess
    import tempfile
    import arena_compaction_amd as ac
    structs = {"defrag_table": ac.defrag_table, "defrag_stats_t": ac.defrag_stats_t,
               "defrag_tuning": ac.defrag_tuning, "defrag_plan_t": ac.defrag_plan_t,
               "defrag_compact_args": ac.defrag_compact_args,
               "defrag_move_report_t": ac.defrag_move_report_t,
               "defrag_monitor_cfg": ac.defrag_monitor_cfg,
               "defrag_monitor_report": ac.defrag_monitor_report}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "arena_compaction.h"',
             'int main(void) {']
    for name, cls in structs.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines.append('return 0; }')
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "layout.c")
        exe = os.path.join(tmp, "layout")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.splitlines())
    for name, cls in structs.items():
        assert int(got[name]) == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(cls, f).offset, f"{name}.{f}"


def test_static_entry_point_refusals_need_no_gpu():
    """defrag_compact_static refuses, before any HIP call, a workspace (its
    scratch stands in for it) and a table whose plan arrays alone exceed the
    static scratch."""
    import arena_compaction_amd as ac
    L = ac.lib
    plan = ac.defrag_plan_t()
    t = ac.defrag_table(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), None, 16)
    args = ac.defrag_compact_args()
    args.table = ctypes.pointer(t)
    args.arena_bytes = 4096
    args.ws_dev = ctypes.c_void_p(0x3000)
    args.ws_bytes = 1 << 20
    assert L.defrag_compact_static(ctypes.byref(args), None, ctypes.byref(plan), None) == \
        ac.DEFRAG_EINVAL
    assert plan.stats.invalid_reason == 6
    args.ws_dev, args.ws_bytes = None, 0
    t.n = 50_000_000   # ~3 GB of plan arrays
    assert L.defrag_compact_static(ctypes.byref(args), None, ctypes.byref(plan), None) == \
        ac.DEFRAG_ETOOBIG
    assert L.defrag_compact_static(ctypes.byref(args), None, None, None) == ac.DEFRAG_EINVAL
    assert ac.defrag_strerror(ac.DEFRAG_ETOOBIG) not in ("ok", "unknown error")
    # the limit the header states: every workload here fits at full size
    assert ac.STATIC_SCRATCH_BYTES == 128 << 20
    assert ac.defrag_workspace_bytes(2_000_000, 4 << 30) <= ac.STATIC_SCRATCH_BYTES

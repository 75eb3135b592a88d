"""Build libarena_compaction.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libarena_compaction.so")
SOURCES = ["api.cpp", "monitor.cpp", "readback.cpp", "plan.hip", "move.hip", "remap.hip",
           "publish.hip", "static.hip"]
ARCH = "gfx950"  # MI355X (CDNA4) only

# No packed-FP32 instructions anywhere in the device code.  hipcc hands the
# feature to the host pass as well, where x86 does not know it and says so
# once per function ("... is not a recognized feature for this target
# (ignoring feature)"); clang cannot forward an option that takes an argument
# to the device pass alone, so that one harmless line is dropped from the
# compiler's output below and everything else is shown.
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra",
    *NO_PACKED_FP32,
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def run_hipcc(cmd) -> None:
    """Run a hipcc command; show its output except the host pass's note
    about the device-only feature; raise on failure."""
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    shown = [ln for ln in p.stdout.splitlines() if ln.strip() != HOST_FEATURE_NOTE]
    if shown:
        print("\n".join(shown), file=sys.stderr, flush=True)
    if p.returncode != 0:
        raise subprocess.CalledProcessError(p.returncode, cmd)


def build(verbose: bool = False, extra_flags=()) -> str:
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    run_hipcc(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, g++), driven over thousands of random small tables by
tests/oracle_sanitize.cpp: any memory error, undefined behaviour or failed
cross-check fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_oracle_under_asan_ubsan():
    d = tempfile.mkdtemp(prefix="oracle_san_")
    try:
        exe = os.path.join(d, "oracle_sanitize")
        subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        os.path.join(HERE, "oracle_sanitize.cpp"),
                        os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", exe], check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, r.stderr[-4000:]
        assert "oracle sanitize run ok" in r.stdout
    finally:
        shutil.rmtree(d, ignore_errors=True)

"""Packed-sequence spans on the host: the clamp that keeps malformed prefix
sums from addressing rows outside the tensors (packed_side, shared with the
kernels through csrc/span.hpp), compiled with g++ under the address and
undefined-behaviour sanitizers.  CPU only; nothing runs on a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_block_wise_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "span_check.cpp")


def test_packed_span_clamp(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "span_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", CSRC, SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout

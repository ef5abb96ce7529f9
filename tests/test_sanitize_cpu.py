"""The C-ABI layer under the host sanitizers: the library is rebuilt with
the address and undefined-behaviour sanitizers on its host code (its GPU
code is built as usual) and tests/test_abi_cpu.py runs against it in a child
process that preloads the sanitizer runtime.  Any sanitizer report aborts
that process and fails this test.  CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_asan_ubsan(tmp_path):
    from exact_block_wise_amd import build
    try:
        runtime = build.asan_runtime()
        lib = build.build(out_dir=str(tmp_path), sanitize=True)
    except RuntimeError as e:  # no hipcc / runtime in this environment
        pytest.skip(str(e))
    # the sanitizer runtime must come first; whatever the environment
    # already preloads stays preloaded after it
    pre = os.environ.get("LD_PRELOAD", "")
    env = {**os.environ, "EXATTN_LIB": lib, "LD_PRELOAD": runtime + (":" + pre if pre else ""),
           "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1"}
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]

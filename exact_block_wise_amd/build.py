"""Build libexattn.so (the C-ABI attention library) for gfx950 with hipcc.

    python -m exact_block_wise_amd.build          # compile into the package

Every HIP source is compiled for gfx950 only; the library is placed next to
this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libexattn.so")
SOURCES = ["abi.hip", "fwd.hip", "bwd.hip", "merge.hip", "short.hip"]

# Per-source flags.  bwd.hip: the dK/dV kernels keep their gradient
# accumulators in AGPRs through inline-assembly products, and a function that
# names AGPRs in inline assembly otherwise gets the AGPR form for every
# matrix product, so the score tiles S and dP would also land in AGPRs and
# cost one v_accvgpr_read per element before the exponentials.  The VGPR form
# leaves them in VGPRs (the dQ kernels of the file compile to the same code).
SOURCE_FLAGS = {"bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-munsafe-fp-atomics",
    # packed fp32 instructions stay off (see the build notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    out = "\n".join(x for x in out.splitlines() if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


# Host-side sanitizers for the C-ABI layer (argument validation, dispatch):
# each flag applies to the host pass only, the GPU code is built as usual.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                  "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The address-sanitizer runtime of hipcc's clang, which a process that
    loads a sanitized library must preload (Python itself is not built with
    it)."""
    out = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm",
                                       "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("address-sanitizer runtime not found")
    return path


def build(verbose: bool = False, out_dir: str | None = None,
          extra_flags: list[str] | None = None, sanitize: bool = False) -> str:
    """Compile every source and link the shared library; returns its path.

    extra_flags are appended to every compile (e.g. -D tile choices).
    sanitize: build the host code with the address and undefined-behaviour
    sanitizers (load it with asan_runtime() preloaded).
    """
    cc = hipcc()
    if sanitize:
        extra_flags = [*SANITIZE_FLAGS, *(extra_flags or [])]
    obj_dir = os.path.join(out_dir or HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        jobs.append((obj, [cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *(extra_flags or []), "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        for out in ex.map(lambda j: _run(j[1]), jobs):
            if verbose and out:
                print(out)
    lib = os.path.join(out_dir, "libexattn.so") if out_dir else LIB
    tmp = lib + ".tmp"
    # every symbol resolved at link time: a missing definition fails the build
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-shared-libsan"] if sanitize else []
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *link_san,
          *([] if sanitize else ["-Wl,--no-undefined"]), *[o for o, _ in jobs], "-o", tmp])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

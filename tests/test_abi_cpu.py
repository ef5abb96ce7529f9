"""The C-ABI library on the CPU: it loads, exports what include/exattn.h
declares, and rejects invalid arguments on the host before any HIP call.

No test here launches a kernel; the fake device pointers below are only
inspected for null-ness and alignment by the library's validation code.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exattn.h")

ebw = pytest.importorskip("exact_block_wise_amd")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ebw.library_path()):
        pytest.fail("libexattn.so is not built (run __graft_entry__.build())")
    return ebw.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "attn_abi_version", "attn_bwd", "attn_bwd_preprocess", "attn_bwd_workspace_bytes",
        "attn_fwd", "attn_fwd_chunked", "attn_lse_merge", "attn_status_string",
        "attn_fwd_varlen", "attn_bwd_varlen", "attn_bwd_varlen_workspace_bytes",
        "attn_bwd_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ebw.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(lib):
    assert lib.attn_abi_version() == ebw.ABI_VERSION
    for st in range(5):
        assert lib.attn_status_string(st).decode().startswith("ATTN_")
    assert b"unknown" in lib.attn_status_string(99)


FAKE = 0x10000000  # 16-byte aligned, never dereferenced on the host


def T(ptr=FAKE, dtype=1, sb=12 * 1568 * 64, sh=1568 * 64, sn=64):
    return ebw._Tensor(ptr, dtype, sb, sh, sn)


def P(B=2, H=3, Nq=196, Nkv=196, d=64, scale=0.125):
    return ebw._Problem(B, H, Nq, Nkv, d, scale)


def fwd(lib, p=None, q=None, k=None, v=None, o=None, lse=FAKE):
    return lib.attn_fwd(None if p is False else ctypes.byref(p or P()), q or T(), k or T(),
                        v or T(), o or T(), lse, None)


def test_fwd_validation(lib):
    assert fwd(lib, p=False) == INVALID
    assert fwd(lib, p=P(B=0)) == INVALID
    assert fwd(lib, p=P(Nkv=0)) == INVALID
    assert fwd(lib, p=P(scale=float("nan"))) == INVALID
    # the bf16 kernels need a positive scale (running maximum over unscaled
    # scores, keys masked with -inf before scaling)
    for bad in (0.0, -0.0, -0.125, -1e-30, float("-inf")):
        assert fwd(lib, p=P(scale=bad)) in (UNSUPPORTED, INVALID)
        assert fwd(lib, p=P(scale=bad, d=96)) in (UNSUPPORTED, INVALID)
    assert fwd(lib, p=P(scale=0.0)) == UNSUPPORTED
    assert fwd(lib, p=P(scale=-0.125)) == UNSUPPORTED
    assert fwd(lib, p=P(d=96)) == UNSUPPORTED
    assert fwd(lib, p=P(d=32)) == UNSUPPORTED
    assert fwd(lib, q=T(ptr=0)) == INVALID
    assert fwd(lib, lse=0) == INVALID
    assert fwd(lib, k=T(dtype=0)) == INVALID            # mixed input dtypes
    assert fwd(lib, q=T(dtype=7)) == INVALID
    assert fwd(lib, q=T(dtype=0), k=T(dtype=0), v=T(dtype=0), o=T(dtype=1)) == INVALID
    assert fwd(lib, q=T(ptr=FAKE + 8)) == UNSUPPORTED   # not 16-byte aligned
    assert fwd(lib, v=T(sn=68)) == UNSUPPORTED          # bf16 row stride not a multiple of 8
    assert fwd(lib, o=T(sh=-64)) == INVALID
    assert fwd(lib, lse=FAKE + 2) == UNSUPPORTED
    assert fwd(lib, k=T(sn=(1 << 23) + 8)) == UNSUPPORTED  # row stride above 16 MiB
    assert fwd(lib, p=P(B=1 << 16, H=1 << 15)) == UNSUPPORTED  # B*H past 32-bit indexing


def test_fwd_chunked_validation(lib):
    def call(n=8, p=None, op=FAKE, lp=FAKE):
        return lib.attn_fwd_chunked(ctypes.byref(p or P()), n, T(), T(), T(), op, lp, None)
    assert call(n=0) == INVALID
    assert call(op=0) == INVALID
    assert call(op=FAKE + 4) == UNSUPPORTED
    assert call(p=P(d=100)) == UNSUPPORTED


def test_merge_validation(lib):
    def call(n=8, B=4, H=32, Nq=128, d=128, op=FAKE, lp=FAKE, o=None, lse=FAKE):
        return lib.attn_lse_merge(n, B, H, Nq, d, op, lp, o or T(), lse, None)
    assert call(n=0) == INVALID
    assert call(Nq=0) == INVALID
    assert call(op=0) == INVALID
    assert call(lse=0) == INVALID
    assert call(d=66) == UNSUPPORTED
    assert call(o=T(ptr=FAKE + 2)) == UNSUPPORTED


def test_workspace_query(lib):
    p = P(B=32, H=12, Nq=1568, Nkv=1568, d=64)
    rows = 32 * 12 * 1568
    rup = lambda x: (x + 255) // 256 * 256
    for flags in (0, 1, 2, 4, 8):
        assert lib.attn_bwd_workspace_bytes(ctypes.byref(p), flags) == rup(rows * 4)
    assert lib.attn_bwd_workspace_bytes(None, 0) == 0
    # a short query block against a long key range: the dQ pass is split over
    # 8 key ranges, whose fp32 partials follow D in the workspace (none when
    # dQ is not computed)
    px = P(B=4, H=32, Nq=128, Nkv=32768, d=128)
    rows_x = 4 * 32 * 128
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(px), 0) == rup(rows_x * 4) + 8 * rows_x * 128 * 4
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(px), 4) == rup(rows_x * 4)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(P(d=96)), 0) == 0


def bwd(lib, p=None, dq=None, flags=0, ws=FAKE, ws_bytes=1 << 40, o=None, dout=None, lse=FAKE):
    return lib.attn_bwd(ctypes.byref(p or P()), T(), T(), T(), o or T(), dout or T(), lse,
                        dq or T(), T(), T(), ws, ws_bytes, flags, None)


def test_bwd_validation(lib):
    assert bwd(lib, flags=16) == INVALID                 # unknown flag
    assert bwd(lib, flags=4 | 8) == INVALID              # nothing to compute
    assert bwd(lib, lse=0) == INVALID
    assert bwd(lib, dout=T(dtype=0)) == INVALID
    assert bwd(lib, dq=T(dtype=1), flags=1) == INVALID   # accumulate needs an fp32 dq
    assert bwd(lib, dq=T(dtype=0), flags=0) == INVALID   # otherwise dq is the input dtype
    assert bwd(lib, ws=0) == WORKSPACE
    assert bwd(lib, ws_bytes=1024) == WORKSPACE
    assert bwd(lib, ws=FAKE + 128) == WORKSPACE          # not 256-byte aligned
    assert bwd(lib, p=P(d=48)) == UNSUPPORTED
    assert bwd(lib, p=P(scale=0.0)) == UNSUPPORTED
    assert bwd(lib, p=P(scale=-1.0)) == UNSUPPORTED
    assert bwd(lib, o=T(dtype=0), dq=T(dtype=0), flags=1, ws_bytes=0) == WORKSPACE


def test_bwd_optional_outputs_validation(lib):
    # with NO_DQ a null dq is allowed, so validation reaches the next check
    null = T(ptr=0)
    assert bwd(lib, dq=null, flags=4, ws=0) == WORKSPACE
    assert bwd(lib, dq=null, flags=0) == INVALID
    # with D_PRECOMPUTED a null o is allowed
    assert bwd(lib, o=null, flags=2, ws=0) == WORKSPACE
    assert bwd(lib, o=null, flags=0) == INVALID


def test_preprocess_validation(lib):
    def call(p=None, o=None, dout=None, dsum=FAKE):
        return lib.attn_bwd_preprocess(ctypes.byref(p or P()), o or T(), dout or T(), dsum, None)
    assert call(dsum=0) == INVALID
    assert call(dsum=FAKE + 2) == UNSUPPORTED
    assert call(o=T(ptr=0)) == INVALID
    assert call(o=T(dtype=1), dout=T(dtype=0)) == INVALID   # f32 dO needs an f32 O
    assert call(p=P(d=40)) == UNSUPPORTED


def VL(n_seq=3, H=4, d=64, max_q=200, max_kv=200, total_q=500, total_kv=500, scale=0.125,
       cu_q=FAKE, cu_kv=FAKE):
    return ebw._Varlen(n_seq, H, d, max_q, max_kv, total_q, total_kv, scale, cu_q, cu_kv)


def PT(ptr=FAKE, dtype=1, sh=64, sn=4 * 64):
    return ebw._Tensor(ptr, dtype, 0, sh, sn)


def test_varlen_validation(lib):
    def fwd_v(p=None, q=None, lse=FAKE):
        return lib.attn_fwd_varlen(None if p is False else ctypes.byref(p or VL()), q or PT(),
                                   PT(), PT(), PT(), lse, None)
    assert fwd_v(p=False) == INVALID
    assert fwd_v(p=VL(n_seq=0)) == INVALID
    assert fwd_v(p=VL(max_q=0)) == INVALID
    assert fwd_v(p=VL(total_q=-1)) == INVALID
    assert fwd_v(p=VL(cu_q=0)) == INVALID
    assert fwd_v(p=VL(cu_kv=0)) == INVALID
    assert fwd_v(p=VL(cu_q=FAKE + 2)) == UNSUPPORTED
    assert fwd_v(p=VL(d=96)) == UNSUPPORTED
    assert fwd_v(p=VL(scale=float("inf"))) == INVALID
    assert fwd_v(p=VL(scale=0.0)) == UNSUPPORTED
    assert fwd_v(p=VL(scale=-0.125)) == UNSUPPORTED
    assert fwd_v(lse=0) == INVALID
    assert fwd_v(q=PT(dtype=0)) == INVALID                       # mixed dtypes
    assert lib.attn_fwd_varlen(ctypes.byref(VL()), PT(dtype=0), PT(dtype=0), PT(dtype=0),
                               PT(dtype=0), FAKE, None) == UNSUPPORTED   # fp32: bf16 only
    # workspace: H * total_q floats for D, rounded up to 256 bytes
    assert lib.attn_bwd_varlen_workspace_bytes(ctypes.byref(VL(H=4, total_q=500))) == 8192
    assert lib.attn_bwd_varlen_workspace_bytes(ctypes.byref(VL(n_seq=0))) == 0

    def bwd_v(flags=0, ws=FAKE, ws_bytes=8192, p=None):
        return lib.attn_bwd_varlen(ctypes.byref(p or VL()), PT(), PT(), PT(), PT(), PT(), FAKE,
                                   PT(), PT(), PT(), ws, ws_bytes, flags, None)
    assert bwd_v(ws_bytes=8191) == WORKSPACE
    assert bwd_v(ws=0) == WORKSPACE
    assert bwd_v(ws=FAKE + 16) == WORKSPACE                      # not 256-byte aligned
    assert bwd_v(flags=4 | 8) == INVALID                         # NO_DQ and NO_DKDV
    assert bwd_v(flags=16) == INVALID
    assert bwd_v(flags=1) == INVALID                             # accumulate needs fp32 dq
    assert bwd_v(p=VL(max_kv=-3)) == INVALID
    assert fwd_v(p=VL(n_seq=1 << 20, H=1 << 12)) == UNSUPPORTED  # sequences * heads too many


def test_bwd_noalloc_validation(lib):
    """Every host-side check of attn_bwd, then the scratch size; all before
    the first GPU call (so they run here, without a GPU)."""
    def call(p=None, flags=0, lse=FAKE, dq=None, dout=None):
        return lib.attn_bwd_noalloc(ctypes.byref(p or P()), T(), T(), T(), T(), dout or T(), lse,
                                    dq or T(), T(), T(), flags, None)
    assert call(flags=16) == INVALID
    assert call(flags=4 | 8) == INVALID
    assert call(lse=0) == INVALID
    assert call(dout=T(dtype=0)) == INVALID
    assert call(dq=T(dtype=1), flags=1) == INVALID
    assert call(p=P(d=48)) == UNSUPPORTED
    assert call(p=P(scale=0.0)) == UNSUPPORTED
    # the workspace must fit the 96 MiB scratch: D alone for 2^25 rows is 128 MiB
    big = P(B=1024, H=32, Nq=1024, Nkv=64)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(big), 0) > ebw.NOALLOC_SCRATCH_BYTES
    assert call(p=big) == WORKSPACE
    # the cross-attention shape's split dQ partials (64 MiB + D) fit
    px = P(B=4, H=32, Nq=128, Nkv=32768, d=128)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(px), 0) <= ebw.NOALLOC_SCRATCH_BYTES

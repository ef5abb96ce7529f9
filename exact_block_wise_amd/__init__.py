"""Exact block-wise softmax attention for MI355X (gfx950).

A thin Python binding over the C-ABI library libexattn.so (declared in
include/exattn.h).  It only marshals arguments: torch tensors provide device
memory and the current HIP stream, and every step of the computation runs in
the library's HIP kernels.  There is no fallback: if the library is missing
or fails to load, every call raises.

    o, lse = fwd(q, k, v)                        # [B,H,N,d] tensors
    dq, dk, dv = bwd(q, k, v, o, do, lse)
    dq, dk, dv = bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv)  # no workspace argument
    o_parts, lse_parts = fwd_chunked(q, k, v, n_chunks=8)
    o, lse = lse_merge(o_parts, lse_parts)
    o, lse = fwd_varlen(q, k, v, cu_q, cu_kv, max_q, max_kv)   # packed [T,H,d]
    dq, dk, dv = bwd_varlen(q, k, v, o, do, lse, cu_q, cu_kv, max_q, max_kv)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # imported first so the library binds to torch's HIP runtime

__all__ = ["fwd", "fwd_chunked", "lse_merge", "bwd", "bwd_preprocess", "bwd_noalloc",
           "bwd_workspace_bytes", "fwd_varlen", "bwd_varlen", "bwd_varlen_workspace_bytes",
           "ExattnError", "library_path", "load", "ABI_VERSION",
           "BWD_DQ_ACCUMULATE", "BWD_D_PRECOMPUTED", "BWD_NO_DQ", "BWD_NO_DKDV"]

ABI_VERSION = 1
BWD_DQ_ACCUMULATE = 1
BWD_D_PRECOMPUTED = 2
BWD_NO_DQ = 4
BWD_NO_DKDV = 8
_F32, _BF16 = 0, 1
_DTYPES = {torch.float32: _F32, torch.bfloat16: _BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))


class ExattnError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call} failed: {message} (status {status})")
        self.status = status


class _Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("sn", ctypes.c_int64)]


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nkv", ctypes.c_int32), ("d", ctypes.c_int32), ("scale", ctypes.c_float)]


class _Varlen(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("max_q", ctypes.c_int32), ("max_kv", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("total_kv", ctypes.c_int64),
                ("scale", ctypes.c_float), ("cu_q", ctypes.c_void_p), ("cu_kv", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return os.environ.get("EXATTN_LIB", os.path.join(_HERE, "libexattn.so"))


def load() -> ctypes.CDLL:
    """Load libexattn.so (once).  Raises if it is missing or mismatched."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ExattnError("load", -1, f"{path} not found; build it with "
                          "`python -m exact_block_wise_amd.build`")
    lib = ctypes.CDLL(path)
    T, P = _Tensor, ctypes.POINTER(_Problem)
    vp, fp, i32, u32, sz = (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                            ctypes.c_uint32, ctypes.c_size_t)
    lib.attn_abi_version.restype = ctypes.c_int
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [P, T, T, T, T, fp, vp]
    lib.attn_fwd_chunked.restype = ctypes.c_int
    lib.attn_fwd_chunked.argtypes = [P, i32, T, T, T, fp, fp, vp]
    lib.attn_lse_merge.restype = ctypes.c_int
    lib.attn_lse_merge.argtypes = [i32, i32, i32, i32, i32, fp, fp, T, fp, vp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [P, u32]
    lib.attn_bwd_preprocess.restype = ctypes.c_int
    lib.attn_bwd_preprocess.argtypes = [P, T, T, fp, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P, T, T, T, T, T, fp, T, T, T, vp, sz, u32, vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [P, T, T, T, T, T, fp, T, T, T, u32, vp]
    V = ctypes.POINTER(_Varlen)
    lib.attn_fwd_varlen.restype = ctypes.c_int
    lib.attn_fwd_varlen.argtypes = [V, T, T, T, T, fp, vp]
    lib.attn_bwd_varlen_workspace_bytes.restype = sz
    lib.attn_bwd_varlen_workspace_bytes.argtypes = [V]
    lib.attn_bwd_varlen.restype = ctypes.c_int
    lib.attn_bwd_varlen.argtypes = [V, T, T, T, T, T, fp, T, T, T, vp, sz, u32, vp]
    if lib.attn_abi_version() != ABI_VERSION:
        raise ExattnError("load", -1, f"ABI version {lib.attn_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def _check(call: str, st: int):
    if st != 0:
        raise ExattnError(call, st, load().attn_status_string(st).decode())


def _desc(t: torch.Tensor) -> _Tensor:
    if t.dim() != 4:
        raise ValueError(f"expected a [B,H,N,d] tensor, got shape {tuple(t.shape)}")
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return _Tensor(t.data_ptr(), _DTYPES[t.dtype], t.stride(0), t.stride(1), t.stride(2))


def _problem(q, k, scale) -> _Problem:
    B, H, Nq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return _Problem(B, H, Nq, k.shape[2], d, scale)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_f32_contig(t, shape, name):
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")


# The C ABI receives pointers and strides, not extents: a tensor smaller than
# the problem it is passed for would be read or written past its end.  So
# every tensor is checked against the others here, before any library call.

def _same_device(**named):
    devs = {n: t.device for n, t in named.items() if t is not None}
    if len(set(devs.values())) > 1:
        raise ValueError("all tensors must be on one device, got " +
                         ", ".join(f"{n}: {d}" for n, d in devs.items()))


def _check_ndim(ndim, **named):
    for n, t in named.items():
        if t is not None and t.dim() != ndim:
            raise ValueError(f"{n} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _check_like(ref_name, ref, **named):
    for n, t in named.items():
        if t is not None and tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(ref.shape)} "
                             f"(the shape of {ref_name})")


def _check_qkv(q, k, v, kv_axis):
    """q [..., Nq, ..., d] against k, v: k and v share one shape, and agree
    with q on every axis but the token axis kv_axis."""
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must have the same shape")
    for ax in range(q.dim()):
        if ax != kv_axis and q.shape[ax] != k.shape[ax]:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} differ on axis {ax}; "
                             "only the token axis may differ")


def _check_dense(q, k, v, o=None, dout=None, dq=None, dk=None, dv=None, **extra):
    _check_ndim(4, q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    _check_qkv(q, k, v, kv_axis=2)
    _check_like("q", q, o=o, dout=dout, dq=dq)
    _check_like("k", k, dk=dk, dv=dv)
    _same_device(q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv, **extra)


def fwd(q, k, v, scale=None, out=None, lse=None, out_dtype=None):
    """Forward pass.  Returns (o [B,H,Nq,d], lse [B,H,Nq] float32)."""
    _check_dense(q, k, v, o=out, lse=lse)
    lib = load()
    B, H, Nq, d = q.shape
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_f32_contig(lse, (B, H, Nq), "lse")
    p = _problem(q, k, scale)
    _check("attn_fwd", lib.attn_fwd(ctypes.byref(p), _desc(q), _desc(k), _desc(v), _desc(out),
                                    lse.data_ptr(), _stream(q.device)))
    return out, lse


def fwd_chunked(q, k, v, n_chunks, scale=None, o_parts=None, lse_parts=None):
    """Per-chunk partials over n_chunks key/value chunks, one launch.

    Returns (o_parts [n,B,H,Nq,d] float32, lse_parts [n,B,H,Nq] float32).
    """
    _check_dense(q, k, v, o_parts=o_parts, lse_parts=lse_parts)
    if n_chunks < 1:
        raise ValueError("n_chunks must be >= 1")
    lib = load()
    B, H, Nq, d = q.shape
    if o_parts is None:
        o_parts = torch.empty((n_chunks, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((n_chunks, B, H, Nq), dtype=torch.float32, device=q.device)
    _check_f32_contig(o_parts, (n_chunks, B, H, Nq, d), "o_parts")
    _check_f32_contig(lse_parts, (n_chunks, B, H, Nq), "lse_parts")
    p = _problem(q, k, scale)
    _check("attn_fwd_chunked",
           lib.attn_fwd_chunked(ctypes.byref(p), n_chunks, _desc(q), _desc(k), _desc(v),
                                o_parts.data_ptr(), lse_parts.data_ptr(), _stream(q.device)))
    return o_parts, lse_parts


def lse_merge(o_parts, lse_parts, out=None, lse=None, out_dtype=torch.bfloat16):
    """Exact merge of partials.  Returns (o [B,H,Nq,d], lse [B,H,Nq])."""
    _check_ndim(5, o_parts=o_parts)
    n, B, H, Nq, d = o_parts.shape
    _check_f32_contig(o_parts, (n, B, H, Nq, d), "o_parts")
    _check_f32_contig(lse_parts, (n, B, H, Nq), "lse_parts")
    if out is not None and tuple(out.shape) != (B, H, Nq, d):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, Nq, d)}")
    _same_device(o_parts=o_parts, lse_parts=lse_parts, out=out, lse=lse)
    lib = load()
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=o_parts.device)
    _check_f32_contig(lse, (B, H, Nq), "lse")
    _check("attn_lse_merge",
           lib.attn_lse_merge(n, B, H, Nq, d, o_parts.data_ptr(), lse_parts.data_ptr(),
                              _desc(out), lse.data_ptr(), _stream(o_parts.device)))
    return out, lse


def bwd_workspace_bytes(q, k, accumulate_dq=False) -> int:
    p = _problem(q, k, None)
    return int(load().attn_bwd_workspace_bytes(ctypes.byref(p),
                                               BWD_DQ_ACCUMULATE if accumulate_dq else 0))


def bwd_preprocess(o, dout, dsum=None):
    """D = rowsum(dO * O) in fp32, [B,H,Nq] (the attn_bwd workspace layout)."""
    _check_ndim(4, o=o, dout=dout)
    _check_like("o", o, dout=dout)
    _same_device(o=o, dout=dout, dsum=dsum)
    lib = load()
    B, H, Nq, d = o.shape
    if dsum is None:
        dsum = torch.empty((B, H, Nq), dtype=torch.float32, device=o.device)
    if dsum.dtype != torch.float32 or not dsum.is_contiguous() or dsum.numel() < B * H * Nq:
        raise ValueError("dsum must be contiguous float32 with at least B*H*Nq elements")
    p = _Problem(B, H, Nq, Nq, d, 1.0)
    _check("attn_bwd_preprocess", lib.attn_bwd_preprocess(ctypes.byref(p), _desc(o), _desc(dout),
                                                          dsum.data_ptr(), _stream(o.device)))
    return dsum


def _desc_or_null(t):
    return _desc(t) if t is not None else _Tensor(None, _BF16, 0, 0, 0)


def bwd(q, k, v, o, dout, lse, scale=None, dq=None, dk=None, dv=None,
        accumulate_dq=False, workspace=None, d_precomputed=False, need_dq=True,
        need_dkdv=True):
    """Backward pass from the saved LSE.  Returns (dq, dk, dv).

    accumulate_dq: the gradient is added to dq, which must be float32 (the
      chunked backward: pass the merged o and lse for every chunk).
    d_precomputed: `workspace` already holds D = rowsum(dO * O) (see
      bwd_preprocess); o may then be None.
    need_dq / need_dkdv: compute only one half (the other outputs are None).
    """
    _check_dense(q, k, v, o=o, dout=dout, dq=dq, dk=dk, dv=dv, lse=lse, workspace=workspace)
    lib = load()
    if need_dq and dq is None:
        dq = (torch.zeros_like(q, dtype=torch.float32) if accumulate_dq else torch.empty_like(q))
    if need_dkdv and dk is None:
        dk = torch.empty_like(k)
    if need_dkdv and dv is None:
        dv = torch.empty_like(v)
    B, H, Nq, d = q.shape
    _check_f32_contig(lse, (B, H, Nq), "lse")
    flags = ((BWD_DQ_ACCUMULATE if accumulate_dq else 0) |
             (BWD_D_PRECOMPUTED if d_precomputed else 0) |
             (0 if need_dq else BWD_NO_DQ) | (0 if need_dkdv else BWD_NO_DKDV))
    p = _problem(q, k, scale)
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p), flags)
    if workspace is None:
        if d_precomputed:
            raise ValueError("d_precomputed needs the workspace that holds D")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("attn_bwd",
           lib.attn_bwd(ctypes.byref(p), _desc(q), _desc(k), _desc(v), _desc_or_null(o),
                        _desc(dout), lse.data_ptr(),
                        _desc_or_null(dq if need_dq else None),
                        _desc_or_null(dk if need_dkdv else None),
                        _desc_or_null(dv if need_dkdv else None),
                        workspace.data_ptr(), ws_bytes, flags, _stream(q.device)))
    return (dq if need_dq else None, dk if need_dkdv else None, dv if need_dkdv else None)


NOALLOC_SCRATCH_BYTES = 96 << 20


def bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale=None, accumulate_dq=False,
                d_precomputed=False, need_dq=True, need_dkdv=True):
    """attn_bwd_noalloc: the backward with the library's own per-GPU scratch
    as workspace (the C call allocates nothing).  The outputs are passed in;
    d_precomputed: the scratch holds D from the previous such call with the
    same o and dout.  Arguments otherwise as bwd.  Returns (dq, dk, dv)."""
    _check_dense(q, k, v, o=o, dout=dout, dq=dq, dk=dk, dv=dv, lse=lse)
    lib = load()
    B, H, Nq, d = q.shape
    _check_f32_contig(lse, (B, H, Nq), "lse")
    flags = ((BWD_DQ_ACCUMULATE if accumulate_dq else 0) |
             (BWD_D_PRECOMPUTED if d_precomputed else 0) |
             (0 if need_dq else BWD_NO_DQ) | (0 if need_dkdv else BWD_NO_DKDV))
    p = _problem(q, k, scale)
    _check("attn_bwd_noalloc",
           lib.attn_bwd_noalloc(ctypes.byref(p), _desc(q), _desc(k), _desc(v), _desc_or_null(o),
                                _desc(dout), lse.data_ptr(),
                                _desc_or_null(dq if need_dq else None),
                                _desc_or_null(dk if need_dkdv else None),
                                _desc_or_null(dv if need_dkdv else None), flags,
                                _stream(q.device)))
    return (dq if need_dq else None, dk if need_dkdv else None, dv if need_dkdv else None)


# --------------------------------------------------------------------------
# Packed variable-length sequences: q, o, dout [Tq, H, d]; k, v [Tkv, H, d];
# cu_q / cu_kv int32 prefix sums on the GPU; lse [H, Tq].
# --------------------------------------------------------------------------

def _packed_desc(t: torch.Tensor) -> _Tensor:
    if t.dim() != 3:
        raise ValueError(f"expected a packed [T,H,d] tensor, got shape {tuple(t.shape)}")
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return _Tensor(t.data_ptr(), _DTYPES[t.dtype], 0, t.stride(1), t.stride(0))


def _packed_desc_or_null(t):
    return _packed_desc(t) if t is not None else _Tensor(None, _BF16, 0, 0, 0)


def _check_packed(q, k, v, o=None, dout=None, dq=None, dk=None, dv=None, **extra):
    _check_ndim(3, q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    _check_qkv(q, k, v, kv_axis=0)
    _check_like("q", q, o=o, dout=dout, dq=dq)
    _check_like("k", k, dk=dk, dv=dv)
    _same_device(q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv, **extra)


def _varlen(q, k, cu_q, cu_kv, max_q, max_kv, scale) -> _Varlen:
    for name, c in (("cu_q", cu_q), ("cu_kv", cu_kv)):
        if c.dtype != torch.int32 or not c.is_cuda or not c.is_contiguous() or c.dim() != 1:
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if cu_q.numel() != cu_kv.numel() or cu_q.numel() < 2:
        raise ValueError("cu_q and cu_kv need n_seq + 1 >= 2 entries each")
    Tq, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return _Varlen(cu_q.numel() - 1, H, d, int(max_q), int(max_kv), Tq, k.shape[0], scale,
                   cu_q.data_ptr(), cu_kv.data_ptr())


def fwd_varlen(q, k, v, cu_q, cu_kv, max_q, max_kv, scale=None, out=None, lse=None,
               out_dtype=None):
    """Forward over packed sequences.  Returns (o [Tq,H,d], lse [H,Tq] float32)."""
    _check_packed(q, k, v, o=out, lse=lse, cu_q=cu_q, cu_kv=cu_kv)
    lib = load()
    Tq, H, d = q.shape
    if out is None:
        out = torch.empty((Tq, H, d), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    _check_f32_contig(lse, (H, Tq), "lse")
    p = _varlen(q, k, cu_q, cu_kv, max_q, max_kv, scale)
    _check("attn_fwd_varlen",
           lib.attn_fwd_varlen(ctypes.byref(p), _packed_desc(q), _packed_desc(k),
                               _packed_desc(v), _packed_desc(out), lse.data_ptr(),
                               _stream(q.device)))
    return out, lse


def bwd_varlen_workspace_bytes(q, k, cu_q, cu_kv, max_q, max_kv) -> int:
    p = _varlen(q, k, cu_q, cu_kv, max_q, max_kv, None)
    return int(load().attn_bwd_varlen_workspace_bytes(ctypes.byref(p)))


def bwd_varlen(q, k, v, o, dout, lse, cu_q, cu_kv, max_q, max_kv, scale=None, dq=None,
               dk=None, dv=None, accumulate_dq=False, workspace=None, d_precomputed=False,
               need_dq=True, need_dkdv=True):
    """Backward over packed sequences; arguments as bwd.  Returns (dq, dk, dv)."""
    _check_packed(q, k, v, o=o, dout=dout, dq=dq, dk=dk, dv=dv, lse=lse, cu_q=cu_q, cu_kv=cu_kv,
                  workspace=workspace)
    lib = load()
    if need_dq and dq is None:
        dq = (torch.zeros_like(q, dtype=torch.float32) if accumulate_dq else torch.empty_like(q))
    if need_dkdv and dk is None:
        dk = torch.empty_like(k)
    if need_dkdv and dv is None:
        dv = torch.empty_like(v)
    Tq, H, d = q.shape
    _check_f32_contig(lse, (H, Tq), "lse")
    flags = ((BWD_DQ_ACCUMULATE if accumulate_dq else 0) |
             (BWD_D_PRECOMPUTED if d_precomputed else 0) |
             (0 if need_dq else BWD_NO_DQ) | (0 if need_dkdv else BWD_NO_DKDV))
    p = _varlen(q, k, cu_q, cu_kv, max_q, max_kv, scale)
    need = lib.attn_bwd_varlen_workspace_bytes(ctypes.byref(p))
    if workspace is None:
        if d_precomputed:
            raise ValueError("d_precomputed needs the workspace that holds D")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("attn_bwd_varlen",
           lib.attn_bwd_varlen(ctypes.byref(p), _packed_desc(q), _packed_desc(k),
                               _packed_desc(v), _packed_desc_or_null(o), _packed_desc(dout),
                               lse.data_ptr(), _packed_desc_or_null(dq if need_dq else None),
                               _packed_desc_or_null(dk if need_dkdv else None),
                               _packed_desc_or_null(dv if need_dkdv else None),
                               workspace.data_ptr(), ws_bytes, flags, _stream(q.device)))
    return (dq if need_dq else None, dk if need_dkdv else None, dv if need_dkdv else None)

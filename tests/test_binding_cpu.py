"""The Python binding rejects tensors that disagree with each other before
any library call.  The C ABI receives pointers and strides but no extents,
so these checks are what keeps a mismatched tensor from being read or
written past its end.  CPU only: meta tensors carry shapes without memory,
and every case here raises before the library is reached."""
import pytest
import torch

import exact_block_wise_amd as ebw


def t(*shape, dtype=torch.bfloat16, device="meta"):
    return torch.empty(shape, dtype=dtype, device=device)


B, H, NQ, NKV, D = 2, 3, 40, 56, 64


def qkv():
    return t(B, H, NQ, D), t(B, H, NKV, D), t(B, H, NKV, D)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_fwd_mismatches():
    q, k, v = qkv()
    raises(lambda: ebw.fwd(q, k, t(B, H, NKV + 1, D)), "same shape")
    raises(lambda: ebw.fwd(q, t(B, H + 1, NKV, D), t(B, H + 1, NKV, D)), "axis 1")
    raises(lambda: ebw.fwd(q, t(B + 1, H, NKV, D), t(B + 1, H, NKV, D)), "axis 0")
    raises(lambda: ebw.fwd(q, t(B, H, NKV, 80), t(B, H, NKV, 80)), "axis 3")
    raises(lambda: ebw.fwd(q, k, v, out=t(B, H, NQ - 1, D)), "expected")
    raises(lambda: ebw.fwd(t(B, H, NQ), k, v), "4 dimensions")
    raises(lambda: ebw.fwd(q, k, v, lse=t(B, H, NQ, dtype=torch.float32, device="cpu")),
           "one device")
    # consistent shapes get past these checks (and then need a GPU)
    raises(lambda: ebw.fwd(q, k, v), "GPU")


def test_fwd_chunked_and_merge_mismatches():
    q, k, v = qkv()
    raises(lambda: ebw.fwd_chunked(q, k, t(B, H, NKV, 80), 4), "same shape")
    raises(lambda: ebw.fwd_chunked(q, k, v, 0), "n_chunks")
    op = t(4, B, H, NQ, D, dtype=torch.float32)
    lp = t(4, B, H, NQ, dtype=torch.float32)
    raises(lambda: ebw.lse_merge(op, t(4, B, H, NQ + 1, dtype=torch.float32)), "lse_parts")
    raises(lambda: ebw.lse_merge(op, lp, out=t(B, H, NQ, D + 16)), "expected")
    raises(lambda: ebw.lse_merge(op, lp, out=t(B, H, NQ, D, device="cpu")), "one device")
    raises(lambda: ebw.lse_merge(t(B, H, NQ, D, dtype=torch.float32), lp), "5 dimensions")


def test_bwd_mismatches():
    q, k, v = qkv()
    o, do = t(B, H, NQ, D), t(B, H, NQ, D)
    lse = t(B, H, NQ, dtype=torch.float32)
    raises(lambda: ebw.bwd(q, k, v, o, t(B, H, NQ + 1, D), lse), "dout")
    raises(lambda: ebw.bwd(q, k, v, t(B, H, NQ, 80), do, lse), "o has shape")
    raises(lambda: ebw.bwd(q, k, v, o, do, lse, dq=t(B, H, NKV, D)), "dq has shape")
    raises(lambda: ebw.bwd(q, k, v, o, do, lse, dk=t(B, H, NQ, D)), "dk has shape")
    raises(lambda: ebw.bwd(q, k, v, o, do, lse, dv=t(B, H, NKV, D + 16)), "dv has shape")
    raises(lambda: ebw.bwd(q, t(B, H, NKV, D), t(B, H, NKV - 8, D), o, do, lse), "same shape")
    raises(lambda: ebw.bwd(q, k, v, o, do, lse,
                           workspace=torch.empty(16, dtype=torch.uint8)), "one device")
    raises(lambda: ebw.bwd_preprocess(o, t(B, H, NQ, 80)), "dout has shape")


def test_varlen_mismatches():
    Tq, Tkv = 100, 120
    q, k, v = t(Tq, H, D), t(Tkv, H, D), t(Tkv, H, D)
    cu = t(4, dtype=torch.int32)
    raises(lambda: ebw.fwd_varlen(q, k, t(Tkv + 1, H, D), cu, cu, 50, 50), "same shape")
    raises(lambda: ebw.fwd_varlen(q, t(Tkv, H + 1, D), t(Tkv, H + 1, D), cu, cu, 50, 50),
           "axis 1")
    raises(lambda: ebw.fwd_varlen(q, k, v, cu, cu, 50, 50, out=t(Tq, H, 80)), "expected")
    raises(lambda: ebw.fwd_varlen(q, k, v, t(4, dtype=torch.int32, device="cpu"), cu, 50, 50),
           "one device")
    o, do = t(Tq, H, D), t(Tq, H, D)
    lse = t(H, Tq, dtype=torch.float32)
    raises(lambda: ebw.bwd_varlen(q, k, v, o, do, lse, cu, cu, 50, 50, dk=t(Tq, H, D)),
           "dk has shape")
    raises(lambda: ebw.bwd_varlen(q, k, v, o, t(Tq - 1, H, D), lse, cu, cu, 50, 50), "dout")

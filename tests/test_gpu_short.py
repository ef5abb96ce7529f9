"""Short sequences (Nq, Nkv <= 32, bf16) against the fp64 oracle (GPU only).

These shapes take the packed-tile kernels, where one 32-row product tile
holds several sequences and scores across sequences are masked off: the
divided space-time attention layers of a video ViT (temporal attention over
t = 8 frames).  Every case is compared element by element; the cases cover
each slot size (8, 16, 32), Nq != Nkv, a last tile only partly filled with
sequences, d = 64 / 80 / 128, strided views, a peaky softmax and every
backward flag.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_block_wise_amd import synth
import full_compare
from gpu_util import TOL_GRAD_FRO, check_fwd, check_grads, max_abs, to_dev, to_host

pytestmark = pytest.mark.gpu

ebw = pytest.importorskip("exact_block_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ebw.load()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def _scale(d):
    return float(np.float32(1 / np.sqrt(d)))


SHORT = [
    # (B, H, Nq, Nkv, d, q_mult)
    (3, 5, 8, 8, 64, 1.0),      # 15 sequences of 8: four per tile, last tile 3/4 full
    (2, 3, 5, 7, 64, 1.0),      # slot 8, Nq != Nkv, ragged slots
    (1, 7, 16, 16, 80, 1.0),    # slot 16, d = 80
    (2, 2, 12, 9, 128, 1.0),    # slot 16, d = 128
    (1, 3, 32, 32, 64, 1.0),    # slot 32: one sequence per tile
    (1, 2, 20, 32, 80, 1.0),    # slot 32, Nq != Nkv
    (4, 1, 1, 8, 64, 1.0),      # one query per sequence
    (2, 2, 8, 1, 64, 1.0),      # one key: O = v_1, dQ = dK = 0
    (5, 3, 8, 8, 64, 8.0),      # peaky softmax
    (3, 2, 16, 16, 128, 8.0),
]


@pytest.mark.parametrize("case", SHORT, ids=lambda c: "x".join(map(str, c[:5])) + f"-q{c[5]:g}")
def test_short_parity(case):
    B, H, Nq, Nkv, d, qm = case
    _say(f"short case {case}")
    x = synth.random_case(zlib.crc32(repr(case).encode()), B, H, Nq, Nkv, d, "bf16", q_mult=qm)
    scale = _scale(d)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v, scale=scale)
    dq, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16")
    check_grads([to_host(t) for t in (dq, dk, dv)],
                oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale), "bf16")


@pytest.mark.parametrize("d", [64, 80, 128])
def test_short_flags_and_outputs(d):
    """NO_DQ / NO_DKDV / precomputed D give the bits of the full call; dQ
    accumulation adds the same values; an fp32 O matches the oracle tightly."""
    B, H, Nq, Nkv = 3, 3, 8, 6
    x = synth.random_case(500 + d, B, H, Nq, Nkv, d, "bf16")
    scale = _scale(d)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v, scale=scale)
    full = ebw.bwd(q, k, v, o, do, lse, scale=scale)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)
    dq, _, _ = ebw.bwd(q, k, v, None, do, lse, scale=scale, workspace=ws, d_precomputed=True,
                       need_dkdv=False)
    _, dk, dv = ebw.bwd(q, k, v, None, do, lse, scale=scale, workspace=ws, d_precomputed=True,
                        need_dq=False)
    # D formed by the backward itself equals the preprocess's D
    ws2 = torch.zeros_like(ws)
    ebw.bwd(q, k, v, o, do, lse, scale=scale, workspace=ws2, need_dkdv=False)
    torch.cuda.synchronize()
    for a_, b_ in zip(full, (dq, dk, dv)):
        assert torch.equal(a_, b_)
    rows = B * H * Nq
    assert max_abs(to_host(ws2[:rows]), to_host(ws[:rows])) < 1e-5
    # accumulation into an fp32 dQ
    base = torch.randn((B, H, Nq, d), dtype=torch.float32, device="cuda")
    acc = base.clone()
    ebw.bwd(q, k, v, o, do, lse, scale=scale, dq=acc, accumulate_dq=True, need_dkdv=False)
    torch.cuda.synchronize()
    ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    got = to_host(acc) - to_host(base)
    check_grads([got, ref[1], ref[2]], ref, "bf16", "accumulated")
    # fp32 output of bf16 inputs (a partial for the merge)
    o32, lse32 = ebw.fwd(q, k, v, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    assert o32.dtype == torch.float32
    assert max_abs(to_host(o32), o_ref) < 4e-3
    assert max_abs(to_host(lse32), lse_ref) < 1e-3
    # the backward from that fp32 O (D from the preprocess kernel)
    g32 = ebw.bwd(q, k, v, o32, do, lse32, scale=scale)
    torch.cuda.synchronize()
    check_grads([to_host(t) for t in g32], ref, "bf16", "from fp32 O")


def test_short_strided_views():
    """Q as a head-strided slice, K and V as column halves of one buffer."""
    B, H, Nq, Nkv, d = 3, 4, 8, 8, 64
    g = np.random.Generator(np.random.PCG64(909))
    big = synth.round_to_bf16(g.standard_normal((B, H + 2, Nq + 3, d), dtype=np.float32))
    kv = synth.round_to_bf16(g.standard_normal((B, H, Nkv + 5, 2 * d), dtype=np.float32))
    do = synth.round_to_bf16(g.standard_normal((B, H, Nq, d), dtype=np.float32))
    qd, kvd = to_dev(big, "bf16"), to_dev(kv, "bf16")
    q = qd[:, 1:H + 1, 2:Nq + 2, :]
    k = kvd[:, :, 3:Nkv + 3, :d]
    v = kvd[:, :, 3:Nkv + 3, d:]
    x = {"q": big[:, 1:H + 1, 2:Nq + 2], "k": kv[:, :, 3:Nkv + 3, :d],
         "v": kv[:, :, 3:Nkv + 3, d:], "do": do}
    scale = _scale(d)
    o, lse = ebw.fwd(q, k, v, scale=scale)
    dq, dk, dv = ebw.bwd(q, k, v, o, to_dev(do, "bf16"), lse, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16")
    check_grads([to_host(t) for t in (dq, dk, dv)],
                oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale), "bf16")


@pytest.mark.parametrize("name", ["vit_b_temporal", "vit_b_spatial"])
def test_divided_space_time_workload(name):
    """The full-size divided space-time layers of the ViT-B clips, in the
    benchmark's launch configuration: every output of every sequence against
    the oracle (75264 temporal sequences of 8 tokens, 3072 spatial ones of
    196)."""
    w = synth.WORKLOADS[name]
    _say(f"full-size {name}: generate and upload")
    host = {n: synth.full_tensor(w.cid, n, w.B, w.H, w.Nq if n in ("q", "do") else w.Nkv, w.d,
                                 w.dtype) for n in ("q", "k", "v", "do")}
    q, k, v, do = (to_dev(host[n], w.dtype) for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v, scale=w.scale)
    dq, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=w.scale)
    torch.cuda.synchronize()
    _say(f"full-size {name}: GPU done")
    errs = full_compare.compare_dense(host, {"bench": {"o": o, "lse": lse, "dq": dq, "dk": dk,
                                                       "dv": dv}}, w.scale, w.dtype,
                                      say=_say)["bench"]
    assert errs.heads == w.B * w.H
    full_compare.log_errors(_say, f"{name}, all {errs.heads} sequences", errs, w.dtype)
    errs.check(w.dtype, name)

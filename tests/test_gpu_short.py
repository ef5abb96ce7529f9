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
    benchmark's launch configuration: invariants over every sequence and all
    outputs of sampled sequences against the oracle."""
    w = synth.WORKLOADS[name]
    _say(f"full-size {name}: upload")
    dev = {}
    for n in ("q", "k", "v", "do"):
        rows = w.Nq if n in ("q", "do") else w.Nkv
        dev[n] = to_dev(synth.full_tensor(w.cid, n, w.B, w.H, rows, w.d, w.dtype), w.dtype)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = ebw.fwd(q, k, v, scale=w.scale)
    dq, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=w.scale)
    torch.cuda.synchronize()
    _say(f"full-size {name}: GPU done")
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    # Per sequence: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, measured as
    # || sum_j x_j || / sum_j || x_j || over the d-vectors.  The sums cancel
    # exactly only in exact arithmetic; with O stored in bf16 (D = dO . O then
    # misses sum_k P dP by the rounding of O) and P, dS rounded to bf16 as
    # matrix-core operands, a NumPy emulation of that rounding on 20000
    # sequences of 8 tokens gives at most 4.4e-3 for dK (a per-coordinate
    # ratio would reach 3e-2 on near-cancelling coordinates).
    def ratio(sum_vec, t):
        return float((sum_vec.norm(dim=-1) / t.float().norm(dim=-1).sum(dim=2).clamp_min(1e-30)).max())
    assert ratio(dk.float().sum(dim=2), dk) < 2e-2
    assert ratio(dv.float().sum(dim=2) - do.float().sum(dim=2), dv) < 2e-2
    g = np.random.Generator(np.random.PCG64(w.cid))
    errs = []
    for i in g.choice(w.B * w.H, size=6, replace=False):
        b, h = int(i) // w.H, int(i) % w.H
        hx = synth.workload_head(w, b, h)
        o_ref, lse_ref = oracle.head_fwd(hx["q"], hx["k"], hx["v"], w.scale)
        check_fwd(to_host(o[b, h]), to_host(lse[b, h]), o_ref, lse_ref, "bf16", f"{name}[{b},{h}]")
        ref = oracle.head_bwd(hx["q"], hx["k"], hx["v"], hx["do"], w.scale)
        errs += check_grads([to_host(t[b, h]) for t in (dq, dk, dv)], ref, "bf16",
                            f"{name}[{b},{h}]")
    _say(f"  sampled grad errors max {max(errs):.2e}")
    assert max(errs) < TOL_GRAD_FRO

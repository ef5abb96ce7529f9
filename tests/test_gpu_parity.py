"""HIP kernels against the fp64 oracle, through the C-ABI (GPU only).

Small cases are compared element by element on every output; the full-size
workloads run in the benchmark's launch configuration and every output of
every head is compared with the oracle (tests/full_compare.py).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_block_wise_amd import synth
import full_compare
from gpu_util import (TOL_GRAD_FRO, check_fwd, check_grads, max_abs, rel_fro, to_dev,
                      to_host)

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


def run_case(x, dtype, scale, check_bwd=True):
    """fwd (+ bwd) on the GPU and in the oracle; returns the error summary."""
    q, k, v, do = (to_dev(x[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    errs = check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, dtype)
    if check_bwd:
        dq, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=scale)
        torch.cuda.synchronize()
        ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
        errs += tuple(check_grads([to_host(t) for t in (dq, dk, dv)], ref, dtype))
    return errs


SMALL = [
    # (B, H, Nq, Nkv, d, dtype, q_mult)
    (1, 2, 196, 196, 64, "bf16", 1.0),     # ragged tail in both directions
    (1, 1, 64, 64, 64, "bf16", 1.0),       # exactly one key tile
    (2, 2, 256, 384, 64, "bf16", 1.0),     # several query and key tiles
    (1, 2, 300, 257, 80, "bf16", 1.0),     # d = 80, ragged
    (1, 2, 130, 700, 128, "bf16", 1.0),    # d = 128, Nq != Nkv
    (1, 1, 1, 1, 64, "bf16", 1.0),         # degenerate: one query, one key
    (1, 2, 33, 1, 64, "bf16", 1.0),        # one key: O = v_1, dQ = dK = 0
    (1, 1, 5, 3000, 64, "bf16", 1.0),      # tiny query block, long keys
    (1, 2, 100, 1000, 128, "bf16", 1.0),   # resident query block, ragged keys, d = 128
    (2, 1, 128, 700, 80, "bf16", 1.0),     # resident query block (full), d = 80
    (1, 2, 200, 200, 64, "bf16", 8.0),     # peaky softmax (running max stress)
    (1, 2, 150, 170, 80, "bf16", 8.0),
    (1, 2, 196, 196, 64, "f32", 1.0),
    (1, 2, 100, 77, 80, "f32", 1.0),
    (1, 1, 70, 130, 128, "f32", 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])) + f"-{c[5]}-q{c[6]:g}")
def test_small_parity(case):
    B, H, Nq, Nkv, d, dtype, qm = case
    _say(f"case {case}")
    x = synth.random_case(zlib.crc32(repr(case).encode()), B, H, Nq, Nkv, d, dtype, q_mult=qm)
    scale = float(np.float32(1 / np.sqrt(d)))
    run_case(x, dtype, scale)


def test_tiny_f32_workload():
    """The fp32 workload (1 x 2 heads, 196 tokens, d = 64) at full size."""
    w = synth.WORKLOADS["tiny_f32"]
    x = {n: synth.full_tensor(w.cid, n, w.B, w.H, w.Nq if n in ("q", "do") else w.Nkv, w.d,
                              w.dtype) for n in ("q", "k", "v", "do")}
    errs = run_case(x, "f32", w.scale)
    _say(f"tiny_f32 errors {errs}")


@pytest.mark.parametrize("B,H,Nq,Nkv,d", [(2, 3, 150, 260, 64), (1, 2, 40, 1100, 64),
                                         (1, 2, 100, 700, 128)])
def test_strided_views(B, H, Nq, Nkv, d):
    """Q as a head-strided slice and K/V as views into wider buffers; the
    short-query cases take the resident-query dK/dV kernel and the split dQ."""
    _say(f"strided {B}x{H}x{Nq}x{Nkv}x{d}")
    g = np.random.Generator(np.random.PCG64(77 + Nkv))
    big = synth.round_to_bf16(g.standard_normal((B, H + 2, Nq + 10, d), dtype=np.float32))
    kv = synth.round_to_bf16(g.standard_normal((B, H, Nkv + 40, 2 * d), dtype=np.float32))
    do = synth.round_to_bf16(g.standard_normal((B, H, Nq, d), dtype=np.float32))
    qd, kvd = to_dev(big, "bf16"), to_dev(kv, "bf16")
    q = qd[:, 1:H + 1, 5:Nq + 5, :]
    k = kvd[:, :, 8:Nkv + 8, :d]
    v = kvd[:, :, 8:Nkv + 8, d:]
    x = {"q": big[:, 1:H + 1, 5:Nq + 5], "k": kv[:, :, 8:Nkv + 8, :d],
         "v": kv[:, :, 8:Nkv + 8, d:], "do": do}
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = ebw.fwd(q, k, v, scale=scale)
    dq, dk, dv = ebw.bwd(q, k, v, o, to_dev(do, "bf16"), lse, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16")
    check_grads([to_host(t) for t in (dq, dk, dv)],
                oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale), "bf16")


def test_fp32_output_of_bf16_inputs():
    x = synth.random_case(5, 1, 2, 100, 300, 128, "bf16")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    scale = float(np.float32(128 ** -0.5))
    o, lse = ebw.fwd(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    assert o.dtype == torch.float32
    # fp32 output of bf16 products: no output rounding, so much tighter than 2e-2
    assert max_abs(to_host(o), o_ref) < 4e-3
    assert max_abs(to_host(lse), lse_ref) < 1e-3
    # the backward from an fp32 O: D formed in the dQ kernel and by the
    # preprocess kernel give the same bits
    full = ebw.bwd(q, k, v, o, do, lse)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)
    split = ebw.bwd(q, k, v, None, do, lse, workspace=ws, d_precomputed=True)
    torch.cuda.synchronize()
    for a_, b_ in zip(full, split):
        assert torch.equal(a_, b_)
    check_grads([to_host(t) for t in full], oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale),
                "bf16", "fp32 O")


@pytest.mark.parametrize("n_chunks,Nkv,d", [(8, 1000, 128), (3, 500, 64), (8, 5, 64), (4, 4096, 80)])
def test_chunked_forward_merge_backward(n_chunks, Nkv, d):
    """KV chunk partials in one launch, exact LSE merge, chunk-by-chunk backward
    with the merged O/LSE and dQ accumulation, against the unsplit oracle.
    With Nkv < n_chunks some chunks are empty (LSE = -inf)."""
    _say(f"chunked n={n_chunks} Nkv={Nkv} d={d}")
    B, H, Nq = 2, 3, 70
    x = synth.random_case(1000 + Nkv + d, B, H, Nq, Nkv, d, "bf16")
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o_parts, lse_parts = ebw.fwd_chunked(q, k, v, n_chunks, scale=scale)
    o, lse = ebw.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    L = -(-Nkv // n_chunks)
    bounds = [min(c * L, Nkv) for c in range(n_chunks)] + [Nkv]
    # every partial against the oracle's partial
    for b in range(B):
        for h in range(H):
            _, _, op_ref, lp_ref = oracle.head_chunked_fwd(x["q"][b, h], x["k"][b, h],
                                                           x["v"][b, h], scale, bounds)
            op, lp = to_host(o_parts[:, b, h]), to_host(lse_parts[:, b, h])
            finite = np.isfinite(lp_ref)
            assert np.array_equal(finite, np.isfinite(lp))
            assert np.all(lp[~finite] == -np.inf) and np.all(op[~finite] == 0)
            assert max_abs(lp[finite], lp_ref[finite]) < 1e-3
            assert max_abs(op[finite], op_ref[finite]) < 4e-3
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "merged")
    # backward chunk by chunk, dK/dV written into views of the full tensors
    dq = torch.zeros((B, H, Nq, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)      # D of the merged output, shared by all chunks
    for c in range(n_chunks):
        lo, hi = bounds[c], bounds[c + 1]
        if hi <= lo:
            continue
        ebw.bwd(q, k[:, :, lo:hi], v[:, :, lo:hi], None, do, lse, scale=scale, dq=dq,
                dk=dk[:, :, lo:hi], dv=dv[:, :, lo:hi], accumulate_dq=True, workspace=ws,
                d_precomputed=True)
    torch.cuda.synchronize()
    ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    check_grads([to_host(t) for t in (dq, dk, dv)], ref, "bf16", "chunked")


def test_merge_kernel_against_oracle():
    g = np.random.Generator(np.random.PCG64(31))
    n, B, H, Nq, d = 5, 2, 3, 40, 80
    op = g.standard_normal((n, B, H, Nq, d)).astype(np.float32)
    lp = (g.standard_normal((n, B, H, Nq)) * 3).astype(np.float32)
    lp[1] = -np.inf                      # an empty chunk everywhere
    lp[:, 0, 0, 7] = -np.inf             # a row with no keys at all
    o, lse = ebw.lse_merge(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.lse_merge(op, lp)
    o_h, l_h = to_host(o), to_host(lse)
    assert l_h[0, 0, 7] == -np.inf and np.all(o_h[0, 0, 7] == 0)
    fin = np.isfinite(lse_ref)
    assert max_abs(l_h[fin], lse_ref[fin]) < 1e-5
    assert max_abs(o_h, o_ref) < 1e-5


def test_results_are_bitwise_reproducible():
    """No atomics anywhere: repeated calls give identical bits."""
    x = synth.random_case(3, 1, 2, 300, 300, 64, "bf16")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o1, l1 = ebw.fwd(q, k, v)
    o2, l2 = ebw.fwd(q, k, v)
    g1 = ebw.bwd(q, k, v, o1, do, l1)
    g2 = ebw.bwd(q, k, v, o1, do, l1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 80, 128])
def test_bwd_flags_split_and_shared_preprocess(d):
    """NO_DQ / NO_DKDV halves and a precomputed D give the same bits as the
    full call."""
    x = synth.random_case(40 + d, 2, 2, 200, 333, d, "bf16")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v)
    full = ebw.bwd(q, k, v, o, do, lse)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)
    dq, _, _ = ebw.bwd(q, k, v, None, do, lse, workspace=ws, d_precomputed=True, need_dkdv=False)
    _, dk, dv = ebw.bwd(q, k, v, None, do, lse, workspace=ws, d_precomputed=True, need_dq=False)
    torch.cuda.synchronize()
    for a, b in zip(full, (dq, dk, dv)):
        assert torch.equal(a, b)
    # the benchmark's order: dQ first, forming D into the workspace, then
    # dK/dV from that D; also the same bits
    ws2 = torch.zeros_like(ws)
    dq2, _, _ = ebw.bwd(q, k, v, o, do, lse, workspace=ws2, need_dkdv=False)
    _, dk2, dv2 = ebw.bwd(q, k, v, None, do, lse, workspace=ws2, d_precomputed=True, need_dq=False)
    torch.cuda.synchronize()
    rows = q.shape[0] * q.shape[1] * q.shape[2]
    assert torch.equal(ws2[:rows], ws[:rows])  # D itself
    for a, b in zip(full, (dq2, dk2, dv2)):
        assert torch.equal(a, b)


# --------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times
# --------------------------------------------------------------------------

def _host_inputs(w):
    return {n: synth.full_tensor(w.cid, n, w.B, w.H, w.Nq if n in ("q", "do") else w.Nkv, w.d,
                                 w.dtype) for n in ("q", "k", "v", "do")}


def _chunk_view_backward(w, q, k, v, do, o, lse):
    """The per-chunk backward the header documents for key/value chunks:
    D once from the merged O, then attn_bwd on each chunk's key/value view
    with DQ_ACCUMULATE | D_PRECOMPUTED (fp32 dQ summed over the chunks; dK,
    dV written into the chunk's rows)."""
    L = -(-w.Nkv // w.chunks)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k[:, :, :L], accumulate_dq=True) // 4,
                     dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)
    for c in range(w.chunks):
        lo, hi = c * L, min((c + 1) * L, w.Nkv)
        ebw.bwd(q, k[:, :, lo:hi], v[:, :, lo:hi], None, do, lse, scale=w.scale, dq=dq,
                dk=dk[:, :, lo:hi], dv=dv[:, :, lo:hi], accumulate_dq=True, workspace=ws,
                d_precomputed=True)
    return dq, dk, dv


@pytest.mark.parametrize("name", ["tiny_f32", "vit_b", "vit_l", "vit_h14", "xattn"])
def test_full_size_workload(name):
    """A full-size workload in the launch configuration the benchmark times,
    every output of EVERY head against the oracle.  For the long-KV
    cross-attention also the chunk-by-chunk backward over its 4096-key views
    (resident-query dK/dV, split-key dQ, accumulating reduce at d = 128)."""
    w = synth.WORKLOADS[name]
    _say(f"full-size {name}: generate and upload")
    host = _host_inputs(w)
    q, k, v, do = (to_dev(host[n], w.dtype) for n in ("q", "k", "v", "do"))
    if w.chunks > 1:
        o_parts, lse_parts = ebw.fwd_chunked(q, k, v, w.chunks, scale=w.scale)
        o, lse = ebw.lse_merge(o_parts, lse_parts)
        del o_parts, lse_parts
    else:
        o, lse = ebw.fwd(q, k, v, scale=w.scale)
    dq, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=w.scale)
    outputs = {"bench": {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}}
    if w.chunks > 1:
        cdq, cdk, cdv = _chunk_view_backward(w, q, k, v, do, o, lse)
        outputs["chunk views"] = {"o": o, "lse": lse, "dq": cdq, "dk": cdk, "dv": cdv}
    torch.cuda.synchronize()
    _say(f"full-size {name}: GPU done")
    del q, k, v, do
    totals = full_compare.compare_dense(host, outputs, w.scale, w.dtype, say=_say)
    for label, errs in totals.items():
        assert errs.heads == w.B * w.H
        full_compare.log_errors(_say, f"{name} [{label}], all {errs.heads} heads", errs, w.dtype)
        errs.check(w.dtype, f"{name} [{label}]")


def test_chunk_view_backward_at_cross_attention_shape():
    """The cross-attention shape's chunk-view backward on a slice of its
    batch (B = 1, H = 2, Nq = 128, d = 128, 8 views of 4096 keys), against the
    unsplit oracle: the resident dK/dV kernel, 8-way split dQ and the
    accumulating reduce."""
    w0 = synth.WORKLOADS["xattn"]
    w = synth.Workload(w0.cid, "xattn_slice", 1, 2, w0.Nq, w0.Nkv, w0.d, w0.dtype, w0.chunks)
    host = _host_inputs(w)
    q, k, v, do = (to_dev(host[n], w.dtype) for n in ("q", "k", "v", "do"))
    o_parts, lse_parts = ebw.fwd_chunked(q, k, v, w.chunks, scale=w.scale)
    o, lse = ebw.lse_merge(o_parts, lse_parts)
    dq, dk, dv = _chunk_view_backward(w, q, k, v, do, o, lse)
    torch.cuda.synchronize()
    errs = full_compare.compare_dense(host, {"c": {"o": o, "lse": lse, "dq": dq, "dk": dk,
                                                   "dv": dv}}, w.scale, w.dtype, say=_say)["c"]
    full_compare.log_errors(_say, "xattn slice, chunk views", errs, w.dtype)
    errs.check(w.dtype, "xattn slice chunk views")


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_chunked_forward_merge_backward(d):
    """fp32 inputs through the chunked forward (the wave-split fp32 kernel
    with a chunk grid dimension), the merge and a chunk-by-chunk backward
    with fp32 dQ accumulation, against the unsplit oracle at the fp32
    tolerance."""
    B, H, Nq, Nkv, n_chunks = 1, 2, 70, 250, 3
    x = synth.random_case(2000 + d, B, H, Nq, Nkv, d, "f32")
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (to_dev(x[n], "f32") for n in ("q", "k", "v", "do"))
    o_parts, lse_parts = ebw.fwd_chunked(q, k, v, n_chunks, scale=scale)
    o, lse = ebw.lse_merge(o_parts, lse_parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "f32", "fp32 merged")
    L = -(-Nkv // n_chunks)
    dq = torch.zeros((B, H, Nq, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)
    for c in range(n_chunks):
        lo, hi = c * L, min((c + 1) * L, Nkv)
        ebw.bwd(q, k[:, :, lo:hi], v[:, :, lo:hi], None, do, lse, scale=scale, dq=dq,
                dk=dk[:, :, lo:hi], dv=dv[:, :, lo:hi], accumulate_dq=True, workspace=ws,
                d_precomputed=True)
    torch.cuda.synchronize()
    ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    check_grads([to_host(t) for t in (dq, dk, dv)], ref, "f32", "fp32 chunked")


def test_fp32_bwd_flags():
    """fp32: the NO_DQ / NO_DKDV halves with a precomputed D give the bits of
    the full call."""
    x = synth.random_case(2100, 2, 2, 150, 90, 80, "f32")
    q, k, v, do = (to_dev(x[n], "f32") for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v)
    full = ebw.bwd(q, k, v, o, do, lse)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    ebw.bwd_preprocess(o, do, ws)
    dq, _, _ = ebw.bwd(q, k, v, None, do, lse, workspace=ws, d_precomputed=True, need_dkdv=False)
    _, dk, dv = ebw.bwd(q, k, v, None, do, lse, workspace=ws, d_precomputed=True, need_dq=False)
    torch.cuda.synchronize()
    for a_, b_ in zip(full, (dq, dk, dv)):
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("B,H,Nq,Nkv,d", [(2, 3, 150, 260, 64), (1, 2, 70, 90, 80),
                                         (1, 2, 40, 1100, 128), (3, 2, 8, 6, 64)])
def test_strided_outputs(B, H, Nq, Nkv, d):
    """O, dQ, dK and dV written into column windows of wider rows (row stride
    d + 24, 8 guard columns on each side): every output path (whole rows
    staged through LDS in the general, resident and short-tile kernels; the
    fp32 dQ accumulation) honours the row stride and writes nothing outside
    its window."""
    _say(f"strided outputs {B}x{H}x{Nq}x{Nkv}x{d}")
    x = synth.random_case(3100 + d + Nq, B, H, Nq, Nkv, d, "bf16")
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    guard = 7.0

    def window(rows, dtype=torch.bfloat16):
        buf = torch.full((B, H, rows, d + 24), guard, dtype=dtype, device="cuda")
        return buf, buf[:, :, :, 8:8 + d]

    ob, o = window(Nq)
    dqb, dq = window(Nq)
    dkb, dk = window(Nkv)
    dvb, dv = window(Nkv)
    accb, acc = window(Nq, torch.float32)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ebw.fwd(q, k, v, scale=scale, out=o, lse=lse)
    ebw.bwd(q, k, v, o, do, lse, scale=scale, dq=dq, dk=dk, dv=dv)
    ebw.bwd(q, k, v, o, do, lse, scale=scale, dq=acc, accumulate_dq=True, need_dkdv=False)
    torch.cuda.synchronize()
    for buf in (ob, dqb, dkb, dvb, accb):
        assert bool((buf[..., :8] == guard).all()) and bool((buf[..., 8 + d:] == guard).all())
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16")
    ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    check_grads([to_host(t) for t in (dq, dk, dv)], ref, "bf16", "strided outputs")
    check_grads([to_host(acc) - guard, ref[1], ref[2]], ref, "bf16", "strided accumulation")


@pytest.mark.parametrize("Nq,Nkv,d", [(150, 260, 64), (8, 8, 64), (100, 700, 128)])
def test_head_offsets_beyond_4gib(Nq, Nkv, d):
    """Every input and output a view whose second head starts 4 GiB + 4 KiB
    after its first: each kernel forms a head's address in 64 bits and its
    32-bit buffer offsets stay within one tile from there.  The three shapes
    take the general kernels, the short-sequence tiles, and the resident
    dK/dV kernel with the split dQ."""
    B, H = 1, 2
    sh = (1 << 31) + 2048  # bf16 elements between the heads
    _say(f"head offsets beyond 4 GiB: {B}x{H}x{Nq}x{Nkv}x{d}")
    x = synth.random_case(4100 + Nq + d, B, H, Nq, Nkv, d, "bf16")
    scale = float(np.float32(1 / np.sqrt(d)))

    def far(rows, data=None):
        base = torch.empty(sh + rows * d, dtype=torch.bfloat16, device="cuda")
        t = base.as_strided((B, H, rows, d), (H * sh, sh, d, 1))
        if data is not None:
            t.copy_(to_dev(data, "bf16"))
        return t

    q, do = far(Nq, x["q"]), far(Nq, x["do"])
    k, v = far(Nkv, x["k"]), far(Nkv, x["v"])
    o, dq, dk, dv = far(Nq), far(Nq), far(Nkv), far(Nkv)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ebw.fwd(q, k, v, scale=scale, out=o, lse=lse)
    ebw.bwd(q, k, v, o, do, lse, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.ref_fwd(x["q"], x["k"], x["v"], scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", "far heads")
    check_grads([to_host(t) for t in (dq, dk, dv)],
                oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale), "bf16", "far heads")
    del q, do, k, v, o, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("accumulate", [False, True])
def test_resident_backward_both_halves(d, accumulate):
    """A short query block against a long key range with both halves in one
    call (the resident-query dK/dV kernel and the split-key dQ pass with its
    ordered reduce), against the oracle; with accumulation into an fp32 dQ
    as well."""
    B, H, Nq, Nkv = 2, 3, 100, 1000
    x = synth.random_case(4200 + d, B, H, Nq, Nkv, d, "bf16")
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v, scale=scale)
    if accumulate:
        base = torch.randn(q.shape, dtype=torch.float32, device="cuda")
        dq = base.clone()
        _, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=scale, dq=dq, accumulate_dq=True)
    else:
        dq, dk, dv = ebw.bwd(q, k, v, o, do, lse, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    got_dq = to_host(dq) - (to_host(base) if accumulate else 0.0)
    errs = check_grads([got_dq, to_host(dk), to_host(dv)], ref, "bf16", f"resident d={d}")
    _say(f"  resident d={d} acc={accumulate}: {['%.2e' % e for e in errs]}")


@pytest.mark.parametrize("d", [64, 80, 128])
def test_row_maximum_rising_in_later_tiles(d):
    """Every query shares a direction u, and two late keys lie along it:
    key 300 (scores up to about 6 above the first tile's maximum, around
    the forward's lazy bound of 8 ln 2) and key 700 (at least 60 above it,
    and for nearly every row more than 90, where weights taken against the
    first tile's maximum would overflow fp32).  Each row's maximum therefore
    rises in the middle of the key sequence, where the forward skips the row
    maxima unless a partial sum shows a weight past its bound: both the skip
    and the rescale run, and a missed rescale would give inf / NaN.

    Forward only: with one key holding nearly all the weight, dQ nearly
    vanishes and is ill-conditioned.  Taking D = dO . O from the bf16-rounded
    O, as the backward does, moves it by about its own size: with key 700 at
    48 u instead, that one rounding gives a relative dQ error of 1.008 in
    fp64, so a relative tolerance on dQ cannot be met here."""
    B, H, Nq, Nkv = 1, 2, 160, 1000
    case = ("rising", d)
    _say(f"case {case}")
    x = synth.random_case(zlib.crc32(repr(case).encode()), B, H, Nq, Nkv, d, "bf16")
    u = np.zeros(d, np.float32)
    u[::3] = 1.0
    u /= np.linalg.norm(u)
    x["q"] = synth.round_to_bf16(x["q"] + 6.0 * u)
    x["k"][:, :, 300] = synth.round_to_bf16(8.0 * u)
    x["k"][:, :, 700] = synth.round_to_bf16(256.0 * u)
    scale = float(np.float32(1 / np.sqrt(d)))
    s700 = scale * np.einsum("bhnd,bhd->bhn", x["q"], x["k"][:, :, 700])
    s_first = scale * np.einsum("bhnd,bhmd->bhnm", x["q"], x["k"][:, :, :64]).max(-1)
    assert np.all(s700 - s_first > 60) and np.mean(s700 - s_first > 90) > 0.95
    run_case(x, "bf16", scale, check_bwd=False)


def test_peaky_rows_over_a_long_key_range():
    """A peaky softmax (q x 8) at d = 128 over 1313 keys, whose rows' maxima
    keep rising across key tiles and whose outputs reach |O| ~ 4.4, where
    the bf16 output alone rounds by up to 0.0156.  The forward may skip a
    tile's row maxima only where they would not have raised its reference;
    a looser rule left the dominant weights rounded and gave O errors of
    0.022 here, past the 2e-2 tolerance (0.014 with the rule as it is)."""
    case = (3, 3, 174, 1313, 128, "bf16", 8.0, False)
    _say(f"case {case}")
    B, H, Nq, Nkv, d, dtype, qm, _ = case
    x = synth.random_case(zlib.crc32(repr(case).encode()), B, H, Nq, Nkv, d, dtype, q_mult=qm)
    scale = float(np.float32(1 / np.sqrt(d)))
    eo, el, *_ = run_case(x, dtype, scale)
    _say(f"  O max abs {eo:.4f}, LSE max abs {el:.2e}")

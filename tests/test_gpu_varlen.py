"""Packed variable-length sequences against the fp64 oracle (GPU only).

Each packed sequence must give exactly what the oracle gives for that
sequence alone (its query rows against its own key/value rows).  The cases
mix long and short sequences, unequal query and key lengths, empty
sequences on either side, all three head dims, both kernel families (the
general tiles and the packed short-sequence tiles) and every backward flag;
equal-length sequences must also reproduce the dense entry points bit for
bit.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_block_wise_amd import synth
import full_compare
from gpu_util import check_grads, max_abs, to_dev, to_host, TOL_LSE_ABS, TOL_O_ABS

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


def make_packed(seed, lq, lk, H, d, q_mult=1.0):
    """Packed q, do [Tq,H,d] and k, v [Tkv,H,d] (bf16 values as fp32)."""
    g = np.random.Generator(np.random.PCG64(seed))
    Tq, Tk = sum(lq), sum(lk)
    x = {}
    for name, T in (("q", Tq), ("k", Tk), ("v", Tk), ("do", Tq)):
        a = g.standard_normal((T, H, d), dtype=np.float32)
        if name == "q":
            a = a * np.float32(q_mult)
        x[name] = synth.round_to_bf16(a)
    return x


def cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def oracle_packed(x, lq, lk, H, d, scale):
    """Per-sequence oracle results assembled in the packed layout."""
    cq, ck = cu(lq), cu(lk)
    Tq, Tk = cq[-1], ck[-1]
    o = np.zeros((Tq, H, d)); lse = np.full((H, Tq), -np.inf)
    dq = np.zeros((Tq, H, d)); dk = np.zeros((Tk, H, d)); dv = np.zeros((Tk, H, d))
    for s in range(len(lq)):
        qs, ks = slice(cq[s], cq[s + 1]), slice(ck[s], ck[s + 1])
        if lq[s] == 0 or lk[s] == 0:
            continue    # no queries: nothing; no keys: O = 0, LSE = -inf, dQ = 0
        for h in range(H):
            q, k, v, do = (x[n][sl, h] for n, sl in (("q", qs), ("k", ks), ("v", ks), ("do", qs)))
            oh, lh = oracle.head_fwd(q, k, v, scale)
            o[qs, h], lse[h, qs] = oh, lh
            gq, gk, gv = oracle.head_bwd(q, k, v, do, scale)
            dq[qs, h], dk[ks, h], dv[ks, h] = gq, gk, gv
    return o, lse, dq, dk, dv


def run_packed(x, lq, lk, H, d, scale, dev=None):
    dev = dev or {n: to_dev(x[n], "bf16") for n in ("q", "k", "v", "do")}
    cq, ck = (torch.from_numpy(cu(l)).cuda() for l in (lq, lk))
    mq, mk = max(max(lq), 1), max(max(lk), 1)
    o, lse = ebw.fwd_varlen(dev["q"], dev["k"], dev["v"], cq, ck, mq, mk, scale=scale)
    dq, dk, dv = ebw.bwd_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cq, ck, mq, mk,
                                scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_packed(got, ref):
    o, lse, dq, dk, dv = (to_host(t) for t in got)
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = ref
    fin = np.isfinite(lse_ref)
    assert np.all(lse[~fin] == -np.inf), "a query without keys must get LSE = -inf"
    assert max_abs(lse[fin], lse_ref[fin]) <= TOL_LSE_ABS
    assert max_abs(o, o_ref) <= TOL_O_ABS
    for t in (o, dq, dk, dv):
        assert np.all(np.isfinite(t))
    return check_grads([dq, dk, dv], [dq_ref, dk_ref, dv_ref], "bf16", "packed")


CASES = [
    # (query lengths, key/value lengths, H, d, q_mult)
    ([200, 1, 65, 0, 333, 64], [150, 7, 65, 12, 0, 300], 3, 64, 1.0),  # empty on either side
    ([100, 257], [130, 40], 2, 80, 1.0),
    ([70, 129, 5], [300, 64, 1], 2, 128, 1.0),
    ([8, 3, 0, 32, 17, 1], [8, 5, 4, 32, 20, 1], 5, 64, 1.0),          # short tiles, slot 32
    ([8, 7, 5, 8, 1, 0, 8], [8, 8, 2, 6, 1, 3, 0], 3, 80, 1.0),         # short tiles, slot 8
    ([12, 16, 9], [16, 3, 16], 2, 128, 1.0),                           # short tiles, slot 16
    ([300, 40], [280, 500], 2, 64, 8.0),                               # peaky softmax
    ([8] * 9, [8] * 9, 2, 64, 8.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{len(c[0])}seq-d{c[3]}-q{c[4]:g}")
def test_packed_parity(case):
    lq, lk, H, d, qm = case
    _say(f"packed case {case}")
    x = make_packed(zlib.crc32(repr(case).encode()), lq, lk, H, d, qm)
    scale = _scale(d)
    got = run_packed(x, lq, lk, H, d, scale)
    errs = check_packed(got, oracle_packed(x, lq, lk, H, d, scale))
    _say(f"  grad errors {['%.2e' % e for e in errs]}")


@pytest.mark.parametrize("n,d", [(200, 64), (24, 80)])
def test_packed_equals_dense(n, d):
    """Equal-length sequences: the packed entry points give the dense ones'
    bits (the same kernels, only the row addressing differs)."""
    B, H = 3, 2
    x = synth.random_case(77 + n + d, B, H, n, n, d, "bf16")
    scale = _scale(d)
    dense = {k: to_dev(v, "bf16") for k, v in x.items()}
    o, lse = ebw.fwd(dense["q"], dense["k"], dense["v"], scale=scale)
    dq, dk, dv = ebw.bwd(dense["q"], dense["k"], dense["v"], o, dense["do"], lse, scale=scale)
    # [B,H,N,d] -> packed [B*N, H, d]
    packed = {k: t.permute(0, 2, 1, 3).reshape(B * n, H, d).contiguous() for k, t in dense.items()}
    lens = [n] * B
    po, plse, pdq, pdk, pdv = run_packed(None, lens, lens, H, d, scale, dev=packed)
    torch.cuda.synchronize()
    unpack = lambda t: t.reshape(B, n, H, d).permute(0, 2, 1, 3)
    for a_, b_ in ((o, po), (dq, pdq), (dk, pdk), (dv, pdv)):
        assert torch.equal(a_, unpack(b_))
    assert torch.equal(lse, plse.reshape(H, B, n).permute(1, 0, 2))


@pytest.mark.parametrize("lq,lk,d", [([200, 70, 0], [150, 300, 9], 64),
                                     ([8, 5, 0, 8], [8, 8, 3, 2], 128)])
def test_packed_flags(lq, lk, d):
    """NO_DQ / NO_DKDV halves with D from attn_bwd_preprocess on the packed
    tensors give the full call's bits; dQ accumulation adds the same dQ."""
    H = 3
    x = make_packed(901 + d, lq, lk, H, d)
    scale = _scale(d)
    dev = {n: to_dev(x[n], "bf16") for n in ("q", "k", "v", "do")}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    cq, ck = (torch.from_numpy(cu(l)).cuda() for l in (lq, lk))
    mq, mk = max(lq), max(lk)
    o, lse = ebw.fwd_varlen(q, k, v, cq, ck, mq, mk, scale=scale)
    full = ebw.bwd_varlen(q, k, v, o, do, lse, cq, ck, mq, mk, scale=scale)
    ws = torch.empty(ebw.bwd_varlen_workspace_bytes(q, k, cq, ck, mq, mk) // 4,
                     dtype=torch.float32, device="cuda")
    # D over the packed tokens: the dense preprocess of one [1, H, Tq, d] problem
    ebw.bwd_preprocess(o.permute(1, 0, 2).unsqueeze(0), do.permute(1, 0, 2).unsqueeze(0), ws)
    dq, _, _ = ebw.bwd_varlen(q, k, v, None, do, lse, cq, ck, mq, mk, scale=scale, workspace=ws,
                              d_precomputed=True, need_dkdv=False)
    _, dk, dv = ebw.bwd_varlen(q, k, v, None, do, lse, cq, ck, mq, mk, scale=scale,
                               workspace=ws, d_precomputed=True, need_dq=False)
    # NO_DQ without a precomputed D runs the preprocess itself
    _, dk2, dv2 = ebw.bwd_varlen(q, k, v, o, do, lse, cq, ck, mq, mk, scale=scale, need_dq=False)
    base = torch.randn(q.shape, dtype=torch.float32, device="cuda")
    acc = base.clone()
    ebw.bwd_varlen(q, k, v, o, do, lse, cq, ck, mq, mk, scale=scale, dq=acc, accumulate_dq=True,
                   need_dkdv=False)
    torch.cuda.synchronize()
    for a_, b_ in zip(full, (dq, dk, dv)):
        assert torch.equal(a_, b_)
    assert torch.equal(full[1], dk2) and torch.equal(full[2], dv2)
    ref = oracle_packed(x, lq, lk, H, d, scale)
    check_grads([to_host(acc) - to_host(base), ref[3], ref[4]], ref[2:], "bf16", "accumulated")
    # an fp32 O (the packed forward's fp32 output): D from the preprocess kernel
    o32, lse32 = ebw.fwd_varlen(q, k, v, cq, ck, mq, mk, scale=scale, out_dtype=torch.float32)
    g32 = ebw.bwd_varlen(q, k, v, o32, do, lse32, cq, ck, mq, mk, scale=scale)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    check_grads([to_host(t) for t in g32], ref[2:], "bf16", "from fp32 O")


def test_packed_workload():
    """The packed mixed image / video batch the benchmark times: every
    (sequence, head) problem against the oracle."""
    w = synth.PACKED_WORKLOADS["vit_b_packed"]
    _say(f"packed workload {w.name}: generate and upload")
    host = {n: synth.packed_tensor(w, n) for n in ("q", "k", "v", "do")}
    dev = {n: to_dev(host[n], "bf16") for n in ("q", "k", "v", "do")}
    cq = torch.from_numpy(w.cu).cuda()
    mx = max(w.lens)
    o, lse = ebw.fwd_varlen(dev["q"], dev["k"], dev["v"], cq, cq, mx, mx, scale=w.scale)
    dq, dk, dv = ebw.bwd_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cq, cq, mx, mx,
                                scale=w.scale)
    torch.cuda.synchronize()
    _say(f"packed workload {w.name}: GPU done")
    errs = full_compare.compare_packed(w, host, {"o": o, "lse": lse, "dq": dq, "dk": dk,
                                                 "dv": dv}, say=_say)
    assert errs.heads == len(w.lens) * w.H
    full_compare.log_errors(_say, f"{w.name}, all {errs.heads} problems", errs, "bf16")
    errs.check("bf16", w.name)

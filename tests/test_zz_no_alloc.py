"""attn_bwd_noalloc (the backward whose workspace is the library's own
per-GPU scratch) against attn_bwd with a caller workspace, through the C
ABI: same kernels, so the same bits, and within the stated tolerances of the
fp64 oracle.  Two calls in a row, the second with a smaller problem (the
scratch keeps the first call's contents), then the split halves sharing D
through the scratch, then a split-key dQ problem."""
import numpy as np
import pytest
import torch

import oracle
from exact_block_wise_amd import synth
from gpu_util import check_fwd, check_grads, to_dev, to_host

pytestmark = pytest.mark.gpu

ebw = pytest.importorskip("exact_block_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ebw.load()
    yield
    torch.cuda.synchronize()


def _case(seed, B, H, Nq, Nkv, d):
    x = synth.random_case(seed, B, H, Nq, Nkv, d, "bf16")
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = ebw.fwd(q, k, v, scale=scale)
    return x, scale, q, k, v, do, o, lse


@pytest.mark.parametrize("shapes", [((2, 3, 300, 257, 64), (1, 2, 100, 90, 80))],
                         ids=["larger-then-smaller"])
def test_noalloc_matches_bwd_two_calls(shapes):
    for i, (B, H, Nq, Nkv, d) in enumerate(shapes):
        print(f"noalloc call {i}: B={B} H={H} Nq={Nq} Nkv={Nkv} d={d}", flush=True)
        x, scale, q, k, v, do, o, lse = _case(700 + i, B, H, Nq, Nkv, d)
        ref = ebw.bwd(q, k, v, o, do, lse, scale=scale)
        got = ebw.bwd_noalloc(q, k, v, o, do, lse, torch.empty_like(q), torch.empty_like(k),
                              torch.empty_like(v), scale=scale)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        g_ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
        check_grads([to_host(t) for t in got], g_ref, "bf16", f"noalloc call {i}")


def test_noalloc_halves_share_d_through_the_scratch():
    x, scale, q, k, v, do, o, lse = _case(720, 1, 2, 200, 333, 64)
    ref = ebw.bwd(q, k, v, o, do, lse, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # dQ first forms D into the scratch; dK/dV then reads it (D_PRECOMPUTED)
    ebw.bwd_noalloc(q, k, v, o, do, lse, dq, None, None, scale=scale, need_dkdv=False)
    ebw.bwd_noalloc(q, k, v, None, do, lse, None, dk, dv, scale=scale, need_dq=False,
                    d_precomputed=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, (dq, dk, dv)):
        assert torch.equal(a, b)


def test_noalloc_split_key_dq_and_accumulate():
    """A short query block against a long key range: the dQ pass splits the
    keys and keeps its fp32 partials in the scratch after D; accumulating
    into an fp32 dQ."""
    x, scale, q, k, v, do, o, lse = _case(730, 1, 2, 128, 4096, 128)
    base = torch.randn(q.shape, dtype=torch.float32, device="cuda")
    acc_ref, acc_got = base.clone(), base.clone()
    dk_r, dv_r = torch.empty_like(k), torch.empty_like(v)
    dk_g, dv_g = torch.empty_like(k), torch.empty_like(v)
    ebw.bwd(q, k, v, o, do, lse, scale=scale, dq=acc_ref, dk=dk_r, dv=dv_r, accumulate_dq=True)
    ebw.bwd_noalloc(q, k, v, o, do, lse, acc_got, dk_g, dv_g, scale=scale, accumulate_dq=True)
    torch.cuda.synchronize()
    assert torch.equal(acc_ref, acc_got)
    assert torch.equal(dk_r, dk_g) and torch.equal(dv_r, dv_g)
    g_ref = oracle.ref_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    check_grads([to_host(acc_got) - to_host(base), to_host(dk_g), to_host(dv_g)], g_ref, "bf16",
                "noalloc split-key dQ")

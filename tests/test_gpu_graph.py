"""The library's calls inside a captured HIP graph (GPU only).

Every entry point validates on the host and only enqueues kernels on the
caller's stream: it allocates nothing, records no memset and never
synchronises, so a training step can capture it in a graph.  The captured
forward + backward (general tiles, short-sequence tiles, chunked forward +
merge + accumulating chunked backward) is replayed several times, with eager
work and synchronisations in between, and every replay must give the bits of
the eager calls on the same inputs.
"""
import numpy as np
import pytest
import torch

from exact_block_wise_amd import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

ebw = pytest.importorskip("exact_block_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ebw.load()
    yield
    torch.cuda.synchronize()


def _inputs(seed, B, H, Nq, Nkv, d):
    x = synth.random_case(seed, B, H, Nq, Nkv, d, "bf16")
    return [to_dev(x[n], "bf16") for n in ("q", "k", "v", "do")]


def _dense_step(q, k, v, do, outs, ws):
    o, lse, dq, dk, dv = outs
    ebw.fwd(q, k, v, out=o, lse=lse)
    ebw.bwd(q, k, v, o, do, lse, dq=dq, workspace=ws, need_dkdv=False)
    ebw.bwd(q, k, v, None, do, lse, dk=dk, dv=dv, workspace=ws, d_precomputed=True,
            need_dq=False)


def _chunked_step(q, k, v, do, outs, ws, n_chunks):
    o_parts, lse_parts, o, lse, dq, dk, dv = outs
    Nkv = k.shape[2]
    L = -(-Nkv // n_chunks)
    ebw.fwd_chunked(q, k, v, n_chunks, o_parts=o_parts, lse_parts=lse_parts)
    ebw.lse_merge(o_parts, lse_parts, out=o, lse=lse)
    dq.zero_()  # a fill kernel, not a memset node
    ebw.bwd_preprocess(o, do, ws)
    for c in range(n_chunks):
        lo, hi = c * L, min((c + 1) * L, Nkv)
        ebw.bwd(q, k[:, :, lo:hi], v[:, :, lo:hi], None, do, lse, dq=dq,
                dk=dk[:, :, lo:hi], dv=dv[:, :, lo:hi], accumulate_dq=True, workspace=ws,
                d_precomputed=True)


@pytest.mark.parametrize("shape,chunks", [((2, 3, 150, 260, 64), 0), ((5, 2, 8, 8, 64), 0),
                                          ((1, 2, 70, 900, 128), 3)])
def test_graph_replay_matches_eager(shape, chunks):
    B, H, Nq, Nkv, d = shape
    print(f"graph case {shape} chunks={chunks}", flush=True)
    q, k, v, do = _inputs(4000 + Nq + d, B, H, Nq, Nkv, d)
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4 + 1, dtype=torch.float32, device="cuda")
    if chunks:
        outs = [torch.empty((chunks, B, H, Nq, d), dtype=torch.float32, device="cuda"),
                torch.empty((chunks, B, H, Nq), dtype=torch.float32, device="cuda"),
                torch.empty_like(q), torch.empty((B, H, Nq), dtype=torch.float32, device="cuda"),
                torch.empty(q.shape, dtype=torch.float32, device="cuda"),
                torch.empty_like(k), torch.empty_like(v)]
        step = lambda: _chunked_step(q, k, v, do, outs, ws, chunks)
    else:
        outs = [torch.empty_like(q), torch.empty((B, H, Nq), dtype=torch.float32, device="cuda"),
                torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        step = lambda: _dense_step(q, k, v, do, outs, ws)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    # capture on a side stream (the graph API's requirement), then replay
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))  # the replay must rewrite every output
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(eager, outs):
            assert torch.equal(a_, b_), f"replay {rep} differs from the eager calls"
        # eager work between replays: the same calls outside the graph
        step()
        torch.cuda.synchronize()
        for a_, b_ in zip(eager, outs):
            assert torch.equal(a_, b_)

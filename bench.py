"""Benchmark: attention forward + backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit_b]

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: the forward (for the long-KV cross-attention
workload: the chunk partials in one launch plus the exact LSE merge) and the
backward from the saved LSE.  Throughput is algorithmic flops (4 units
forward + 10 units backward, one unit = B*H*Nq*Nkv*d multiply-adds... counted
as flops below) over wall time measured with HIP events on the stream the
library launches on.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="vit_b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


def upload(w, torch):
    from exact_block_wise_amd import synth
    dev = {}
    for n in ("q", "k", "v", "do"):
        nrows = w.Nq if n in ("q", "do") else w.Nkv
        host = synth.full_tensor(w.cid, n, w.B, w.H, nrows, w.d, w.dtype)
        if w.dtype == "bf16":
            dev[n] = torch.from_numpy(synth.bf16_bits(host)).view(torch.bfloat16).cuda()
        else:
            dev[n] = torch.from_numpy(host).cuda()
        del host
    return dev


def cpu_baseline(w, budget_s):
    """The fp64 oracle on the host cores, over whole heads of the same
    workload until about budget_s seconds of work; scaled to TFLOP/s."""
    import oracle
    from exact_block_wise_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i["num_threads"] for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    heads, t_work = 0, 0.0
    per_head = 14.0 * w.Nq * w.Nkv * w.d
    order = [(b, h) for b in range(w.B) for h in range(w.H)]
    while t_work < budget_s and heads < len(order):
        b, h = order[heads]
        x = synth.workload_head(w, b, h)
        t0 = time.perf_counter()
        if w.chunks > 1:
            L = w.Nkv // w.chunks
            o, lse, _, _ = oracle.head_chunked_fwd(x["q"], x["k"], x["v"], w.scale,
                                                   list(range(0, w.Nkv + 1, L)))
            oracle.head_chunked_bwd(x["q"], x["k"], x["v"], x["do"], w.scale,
                                    list(range(0, w.Nkv + 1, L)), o, lse)
        else:
            oracle.head_fwd(x["q"], x["k"], x["v"], w.scale)
            oracle.head_bwd(x["q"], x["k"], x["v"], x["do"], w.scale)
        t_work += time.perf_counter() - t0
        heads += 1
    return {"value": round(per_head * heads / t_work / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads (b,h) of {w.name}, fwd+bwd in fp64 "
                      f"NumPy, {t_work:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import exact_block_wise_amd as ebw
    from exact_block_wise_amd import synth

    w = synth.WORKLOADS[args.workload]
    dev = upload(w, torch)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    tdt = q.dtype
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=tdt, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(ebw.bwd_workspace_bytes(q, k), 1), dtype=torch.uint8, device="cuda")
    if w.chunks > 1:
        o_parts = torch.empty((w.chunks, w.B, w.H, w.Nq, w.d), dtype=torch.float32, device="cuda")
        lse_parts = torch.empty((w.chunks, w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

    def forward():
        if w.chunks > 1:
            ebw.fwd_chunked(q, k, v, w.chunks, scale=w.scale, o_parts=o_parts, lse_parts=lse_parts)
            ebw.lse_merge(o_parts, lse_parts, out=o, lse=lse)
        else:
            ebw.fwd(q, k, v, scale=w.scale, out=o, lse=lse)

    def backward():
        ebw.bwd(q, k, v, o, do, lse, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(args.warmup):
        forward()
        backward()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        ev[i][0].record()
        forward()
        ev[i][1].record()
        backward()
        ev[i][2].record()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    ms = total_ms / K

    u = float(w.units)
    flops = 14.0 * u
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    bwd_avg = float(np.mean(bwd_ms))
    fwd_avg = float(np.mean(fwd_ms))
    bwd_tflops = 10.0 * u / (bwd_avg * 1e-3) / 1e12
    fwd_tflops = 4.0 * u / (fwd_avg * 1e-3) / 1e12

    line = {
        "metric": "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak, video ViT-B N=1568",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) per head, rounded to the compute dtype",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nkv": w.Nkv, "d": w.d,
                   "kv_chunks": w.chunks, "scale": w.scale},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "fwd_ms": round(fwd_avg, 5),
        "bwd_ms": round(bwd_avg, 5),
        "fwd_tflops": round(fwd_tflops, 3),
        "bwd_tflops": round(bwd_tflops, 3),
        "roofline": {
            "kernel": "attn_bwd (D preprocess + key/value-outer main + dQ cast)",
            "bound": "mfma", "achieved": round(bwd_tflops, 3), "peak": peak,
            "unit": "TFLOP/s", "frac": round(bwd_tflops / peak, 4), "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

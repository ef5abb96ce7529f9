"""Benchmark: attention forward + backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit_b]

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: the forward (for the long-KV cross-attention
workload: the chunk partials in one launch plus the exact LSE merge) and the
backward from the saved LSE.  Throughput is algorithmic flops over wall time
measured with HIP events on the stream the library launches on: with one unit
u = B*H*Nq*Nkv*d, the forward's two matrix products are 4u flops and the
backward's five are 10u.  Prints one JSON line.
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
    ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    if w.chunks > 1:
        o_parts = torch.empty((w.chunks, w.B, w.H, w.Nq, w.d), dtype=torch.float32, device="cuda")
        lse_parts = torch.empty((w.chunks, w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

    # The step, as single-kernel library calls (HIP events between the calls
    # therefore time one kernel each).  Credited flops per call, in units of
    # B*H*Nq*Nkv*d: forward 4; dK/dV 8 (S, dP, dV, dK); dQ 2 (dQ; its S and
    # dP recomputation, 4 more, is extra work and not credited).
    calls = []
    if w.chunks > 1:
        calls.append(("fwd_chunked", 4.0, 4.0, lambda: ebw.fwd_chunked(
            q, k, v, w.chunks, scale=w.scale, o_parts=o_parts, lse_parts=lse_parts)))
        calls.append(("lse_merge", 0.0, 0.0,
                      lambda: ebw.lse_merge(o_parts, lse_parts, out=o, lse=lse)))
    else:
        calls.append(("fwd", 4.0, 4.0,
                      lambda: ebw.fwd(q, k, v, scale=w.scale, out=o, lse=lse)))
    calls.append(("bwd_preprocess", 0.0, 0.0, lambda: ebw.bwd_preprocess(o, do, ws)))
    calls.append(("bwd_dkdv", 8.0, 8.0, lambda: ebw.bwd(
        q, k, v, None, do, lse, scale=w.scale, dk=dk, dv=dv, workspace=ws,
        d_precomputed=True, need_dq=False)))
    calls.append(("bwd_dq", 2.0, 6.0, lambda: ebw.bwd(
        q, k, v, None, do, lse, scale=w.scale, dq=dq, workspace=ws, d_precomputed=True,
        need_dkdv=False)))

    for _ in range(args.warmup):
        for c in calls:
            c[3]()
    torch.cuda.synchronize()

    K = args.steps
    n = len(calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        for j, c in enumerate(calls):
            c[3]()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    total_ms = ev[0][0].elapsed_time(ev[K - 1][n])
    per_call = {c[0]: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]))
                for j, c in enumerate(calls)}
    ms = total_ms / K

    u = float(w.units)
    flops = 14.0 * u
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    fwd_ms = sum(per_call[c[0]] for c in calls if c[0] in ("fwd", "fwd_chunked", "lse_merge"))
    bwd_ms = ms - fwd_ms
    kernels = {}
    for name, credit, executed, _ in calls:
        t = per_call[name]
        kernels[name] = {"ms": round(t, 5)}
        if credit:
            kernels[name]["tflops"] = round(credit * u / (t * 1e-3) / 1e12, 3)
            kernels[name]["executed_tflops"] = round(executed * u / (t * 1e-3) / 1e12, 3)
    dom = max((c for c in calls if c[1] > 0), key=lambda c: per_call[c[0]])
    dom_t = per_call[dom[0]]
    if w.chunks > 1:
        # long-KV cross-attention: HBM-bound; algorithmic bytes of the kernel
        bpe = 2
        kv_bytes = 2 * w.B * w.H * w.Nkv * w.d * bpe
        q_bytes = w.B * w.H * w.Nq * w.d * bpe
        alg = {"fwd_chunked": kv_bytes + q_bytes,
               "bwd_dkdv": 2 * kv_bytes + 2 * q_bytes + 2 * w.B * w.H * w.Nq * 4,
               "bwd_dq": 2 * q_bytes + q_bytes + 2 * w.B * w.H * w.Nq * 4}[dom[0]]
        achieved = alg / (dom_t * 1e-3) / 1e9
        roof = {"kernel": dom[0], "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None}
    else:
        achieved = dom[1] * u / (dom_t * 1e-3) / 1e12
        roof = {"kernel": dom[0], "bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None}

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
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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

import hashlib
import glob
import csv

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: the ViT-B headline line, with every "
                         "other workload summarised under other_workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle work for the headline workload's CPU baseline")
    ap.add_argument("--other-cpu-seconds", type=float, default=4.0,
                    help="oracle work for each other workload's CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for the HBM "
                         "counter scale factors)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time only plain bf16 GEMMs through the vendor library (torch.matmul / "
                         "hipBLASLt): the matrix-core rate this GPU sustains outside attention")
    ap.add_argument("--make-mfma-profile", metavar="PMC_DIR",
                    help="turn a rocprofv3 --pmc run with the matrix-core counters (see "
                         "MFMA_COUNTERS) into profiles/*_mfma_utilisation.txt (workload "
                         "gemm_ceiling: a run of --gemm-ceiling)")
    ap.add_argument("--make-traffic-profile", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                    "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE results of a bench run "
                         "and of a --copy-calibration run into profiles/*_traffic.txt")
    return ap.parse_args()


# --------------------------------------------------------------------------
# HBM traffic of the dominant kernel, from hardware counters
# --------------------------------------------------------------------------
KERNEL_SOURCES = {"fwd": "fwd.hip", "fwd_chunked": "fwd.hip", "bwd_dkdv": "bwd.hip",
                  "bwd_dq": "bwd.hip", "bwd": "short.hip"}
KERNEL_SYMBOLS = {"fwd": "fwd_", "fwd_chunked": "fwd_", "bwd_dkdv": "dkdv_",
                  "bwd_dq": "dq_bf16_kernel", "bwd": "bwd_short_kernel"}
COPY_BYTES = 1 << 31  # 2 GiB read and 2 GiB written by the calibration copy


def is_packed(w):
    """Variable-length sequences packed along one token axis."""
    return hasattr(w, "lens")


def is_short(w):
    """Short sequences (both sides <= 32 rows, bf16): served by the
    packed-tile kernels, whose backward is one call."""
    return (not is_packed(w) and w.dtype == "bf16" and w.chunks == 1 and w.Nq <= 32
            and w.Nkv <= 32)


def find_workload(name):
    from exact_block_wise_amd import synth
    if name in synth.PACKED_WORKLOADS:
        return synth.PACKED_WORKLOADS[name]
    return synth.WORKLOADS[name]


def _code_only(text):
    """Source text without // comments and blank lines (a comment edit does
    not change the kernel)."""
    out = []
    for ln in text.splitlines():
        code = ln.split("//", 1)[0].rstrip()
        if code:
            out.append(code)
    return "\n".join(out)


def source_digest(call, short=False):
    """Digest of the code (comments excluded) of the source a call's kernels
    come from, with the shared header."""
    src = "short.hip" if short else KERNEL_SOURCES[call]
    path = os.path.join(ROOT, "exact_block_wise_amd", "csrc", src)
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "exact_block_wise_amd", "csrc", "common.hpp")):
        h.update(_code_only(open(p, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def copy_calibration():
    """A plain copy of COPY_BYTES (read once, written once), repeated; also
    reports the rate it sustains (bytes read plus written per second, HIP
    events), the HBM rate a streaming kernel reaches on this GPU in practice
    next to the published 8 TB/s."""
    import torch
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes": COPY_BYTES, "ms_per_copy": round(ms, 5),
                      "copy_GBps": round(2 * COPY_BYTES / ms / 1e6, 1),
                      "frac_of_8TBps": round(2 * COPY_BYTES / ms / 1e6 / PEAK_HBM_GBS, 3)}))


def gemm_ceiling():
    """Sustained bf16 rate of plain square GEMMs through the vendor library
    (torch.matmul, hipBLASLt on ROCm), timed with HIP events: the practical
    matrix-core ceiling of this GPU next to the published dense peak."""
    import torch
    torch.manual_seed(0)
    out = {}
    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        it = 20 if n == 16384 else 50
        for _ in range(5):
            a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(it):
            a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / it
        out[f"gemm_{n}"] = {"ms": round(ms, 4), "tflops": round(2 * n ** 3 / ms / 1e9, 1),
                            "frac_of_peak": round(2 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS, 3)}
        del a, b
    print(json.dumps({"gemm_ceiling_bf16": out, "peak_tflops": PEAK_BF16_TFLOPS}))


def _pmc_per_dispatch(d, counter, name_part):
    """Mean per-dispatch value of `counter` (summed over instances) for the
    kernels whose name contains name_part, from a rocprofv3 --pmc csv dir."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
                continue
            key = (f, r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for '{name_part}' under {d}")
    vals = sorted(per.values())
    return vals[len(vals) // 2]


def make_traffic_profile(dirs, workload):
    short = is_short(find_workload(workload))
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    cf = _pmc_per_dispatch(cfetch_dir, "FETCH_SIZE", "copy") * 1024 / COPY_BYTES
    cw = _pmc_per_dispatch(cwrite_dir, "WRITE_SIZE", "copy") * 1024 / COPY_BYTES
    lines = []
    for call, sym in KERNEL_SYMBOLS.items():
        try:
            fk = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", sym)
            wk = _pmc_per_dispatch(write_dir, "WRITE_SIZE", sym)
        except SystemExit:
            continue
        traffic = fk * 1024 / cf + wk * 1024 / cw
        lines.append(f"{call} source={source_digest(call, short)} fetch_kib={fk:.1f} "
                     f"write_kib={wk:.1f} "
                     f"traffic_bytes={traffic:.0f}")
    out = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    with open(out, "w") as f:
        f.write(f"# HBM traffic per dispatch, workload {workload}, from rocprofv3 --pmc\n")
        f.write("# commands (repo root, MI355X), each counter in its own run:\n")
        f.write(f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -- python bench.py "
                f"--workload {workload} --steps 1 --warmup 1 --no-cpu-baseline\n")
        f.write("#   (same with WRITE_SIZE into <W>)\n")
        f.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <CF> -- python bench.py "
                "--copy-calibration   (and WRITE_SIZE into <CW>)\n")
        f.write("#   python bench.py --workload %s --make-traffic-profile <F> <W> <CF> <CW>\n"
                % workload)
        f.write(f"# copy calibration: {COPY_BYTES} bytes read and written; counter/bytes "
                f"factors fetch={cf:.4f} write={cw:.4f}\n")
        f.write("# traffic_bytes = fetch_kib*1024/fetch_factor + write_kib*1024/write_factor;\n")
        f.write("# source = digest of the kernel's source code, comments excluded, when measured\n")
        f.write("# (the bench reports the traffic only while that code is unchanged)\n")
        f.write(f"copy_fetch_factor={cf:.6f} copy_write_factor={cw:.6f}\n")
        for ln in lines:
            f.write(ln + "\n")
    print(open(out).read())


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"


def make_mfma_profile(d, workload):
    """Matrix-core utilisation per kernel from one rocprofv3 run with
    --pmc MFMA_COUNTERS: busy fraction = SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) /
    (GRBM_GUI_ACTIVE per XCD x SIMD count); executed matrix flops =
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; shader clock while the kernel runs =
    GRBM_GUI_ACTIVE per XCD / the dispatch's duration."""
    gemm = workload == "gemm_ceiling"  # the run of --gemm-ceiling
    w = None if gemm else find_workload(workload)
    agent = [r for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True)
             for r in csv.DictReader(open(f)) if r.get("Name", "").startswith("gfx")][0]
    simds, cus, fmax = int(agent["Simd_Count"]), int(agent["Cu_Count"]), int(
        agent["Max_Engine_Clk_Fcompute"])
    xcds = int(agent.get("Num_Xcc") or 1)
    dur = {}
    acc = {}  # (dir, dispatch) -> counter -> value (rocprofv3 sums the instances)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            key = (f.rsplit("/", 1)[0], r["Dispatch_Id"])
            acc.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            dur[key] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    units = 0 if gemm else (w.B * w.H * w.Nq * w.Nkv * w.d if not is_packed(w) else sum(
        n * n for n in w.lens) * w.H * w.d)
    credit = {"fwd_": 4.0, "dq_bf16_kernel": 6.0, "dkdv_": 8.0}
    rows = {}
    for key, cs in acc.items():
        if key not in dur or "GRBM_GUI_ACTIVE" not in cs:
            continue
        name, ns = dur[key]
        if "Cijk" in name:  # the vendor GEMM of --gemm-ceiling: tagged by its shape
            name = "hipBLASLt GEMM (" + name[:40] + "...)"
        elif not any(s_ in name for s_ in credit):
            continue
        # GRBM_GUI_ACTIVE comes summed over the XCDs: the shader clock counts
        # of one XCD are that over the XCD count
        busy, grbm = cs["SQ_VALU_MFMA_BUSY_CYCLES"], cs["GRBM_GUI_ACTIVE"] / xcds
        mops = cs["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
        if name.startswith("hipBLASLt"):
            n_ = round((mops * 512 / 2) ** (1 / 3))  # square n x n x n
            name = f"hipBLASLt bf16 GEMM n={n_}"
        rows.setdefault(name, []).append((busy / (grbm * simds), mops * 512, grbm / ns, ns))
    stem = "bf16_gemm_ceiling" if gemm else workload
    run = "--gemm-ceiling" if gemm else f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline"
    out = os.path.join(ROOT, "profiles", f"{stem}_mfma_utilisation.txt")
    with open(out, "w") as f:
        f.write(f"# matrix-core utilisation per kernel, {'the vendor GEMMs of --gemm-ceiling' if gemm else 'workload ' + workload}, from rocprofv3 --pmc\n")
        f.write("# command (repo root, MI355X):\n")
        f.write(f"#   rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace --output-format csv -d <D> "
                f"-- python bench.py {run}\n")
        f.write(f"#   python bench.py --workload {workload} --make-mfma-profile <D>\n")
        f.write(f"# device (rocprofv3 agent info): {agent['Name']}, {cus} CUs, {simds} SIMDs, "
                f"max shader clock {fmax} MHz\n")
        f.write(f"# GRBM_GUI_ACTIVE as written is summed over the {xcds} XCDs; per XCD = value / "
                f"{xcds}.\n")
        f.write("# busy = SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) / (GRBM_GUI_ACTIVE per XCD x SIMDs);\n")
        f.write("# clock = GRBM_GUI_ACTIVE per XCD / duration (the dispatch's timestamps);\n")
        f.write("# executed flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (padding included: at d = 80\n"
                "# the products run on 96 columns); design = the flops of the kernel's products at\n"
                "# the true d (forward 4u, dQ 6u with its S and dP recomputation, dK/dV 8u, where\n"
                "# u = B*H*Nq*Nkv*d; the bench line credits dQ with 2u only).\n")
        f.write("# Means over the run's dispatches; counter collection serialises kernels, so the\n"
                "# durations are not the bench's.  peak@clock = 2.5 PFLOP/s x clock / max clock.\n")
        f.write(f"{'kernel':58s} {'disp':>4s} {'busy':>6s} {'clock_MHz':>9s} {'exec_GF':>8s} "
                f"{'design_GF':>9s} {'exec_TF/s':>9s} {'peak@clock':>10s}\n")
        for name, rs in sorted(rows.items()):
            n = len(rs)
            busy = sum(r[0] for r in rs) / n
            fl = sum(r[1] for r in rs) / n
            clk = sum(r[2] for r in rs) / n * 1e3
            ns = sum(r[3] for r in rs) / n
            cred = next((credit[s_] * units / 1e9 for s_ in credit if s_ in name), None)
            cred_s = f"{cred:9.1f}" if cred is not None else f"{'-':>9s}"
            f.write(f"{name[:58]:58s} {n:4d} {busy:6.3f} {clk:9.0f} {fl / 1e9:8.1f} "
                    f"{cred_s} {fl / ns / 1e3:9.1f} {PEAK_BF16_TFLOPS * clk / fmax:10.1f}\n")
    print(open(out).read())


def measured_traffic(call, workload, short=False):
    """traffic_bytes of `call` from profiles/, or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    for ln in open(path):
        if ln.startswith(call + " "):
            kv = dict(x.split("=", 1) for x in ln.split()[1:])
            if kv.get("source") == source_digest(call, short):
                return int(float(kv["traffic_bytes"]))
    return None


def upload(w, torch):
    from exact_block_wise_amd import synth
    dev = {}
    if is_packed(w):
        for n in ("q", "k", "v", "do"):
            host = synth.packed_tensor(w, n)
            dev[n] = torch.from_numpy(synth.bf16_bits(host)).view(torch.bfloat16).cuda()
            del host
        dev["cu"] = torch.from_numpy(w.cu).cuda()
        return dev
    for n in ("q", "k", "v", "do"):
        nrows = w.Nq if n in ("q", "do") else w.Nkv
        host = synth.full_tensor(w.cid, n, w.B, w.H, nrows, w.d, w.dtype)
        if w.dtype == "bf16":
            dev[n] = torch.from_numpy(synth.bf16_bits(host)).view(torch.bfloat16).cuda()
        else:
            dev[n] = torch.from_numpy(host).cuda()
        del host
    return dev


def _oracle_head_inputs(w, b, h):
    from exact_block_wise_amd import synth
    if is_packed(w):
        n = w.lens[b]
        return {t: synth.head_tensor(w.cid, t, b, h, w.H, n, w.d, w.dtype)
                for t in ("q", "k", "v", "do")}
    return synth.workload_head(w, b, h)


def _gpu_head(w, outs, b, h):
    """One head's outputs from the GPU results, as float64 host arrays."""
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    if is_packed(w):
        r0, r1 = int(w.cu[b]), int(w.cu[b + 1])
        return {"o": f(outs["o"][r0:r1, h]), "lse": f(outs["lse"][h, r0:r1]),
                **{n: f(outs[n][r0:r1, h]) for n in ("dq", "dk", "dv")}}
    return {n: f(outs[n][b, h]) for n in ("o", "lse", "dq", "dk", "dv")}


def cpu_baseline(w, budget_s, outs=None, repeats=1):
    """The fp64 oracle on the host cores, over whole heads of the same
    workload until about budget_s seconds of work; scaled to TFLOP/s.
    With the GPU outputs of the step (outs), the same oracle results also
    give the GPU's errors on those heads (outside any timed region).  With
    repeats > 1 the sample is timed that many times and the median taken."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i["num_threads"] for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    if is_packed(w):
        order = [(s_, h) for s_ in range(len(w.lens)) for h in range(w.H)]
    else:
        order = [(b, h) for b in range(w.B) for h in range(w.H)]
    # spread the sample over the batch: heads taken with a stride
    stride = max(1, len(order) // 64)
    order = order[::stride] + [x for i, x in enumerate(order) if i % stride]
    err = {"max_abs": {}, "max_ref": {}, "sq_diff": {}, "sq_ref": {}}
    heads, t_work, flops, times = 0, 0.0, 0.0, []
    while heads < len(order) and (t_work < budget_s or heads == 0):
        b, h = order[heads]
        x = _oracle_head_inputs(w, b, h)
        n_q, n_kv = (w.lens[b], w.lens[b]) if is_packed(w) else (w.Nq, w.Nkv)
        flops += 14.0 * n_q * n_kv * w.d
        per = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            if w.chunks > 1:
                L = w.Nkv // w.chunks
                bounds = list(range(0, w.Nkv + 1, L))
                o, lse, _, _ = oracle.head_chunked_fwd(x["q"], x["k"], x["v"], w.scale, bounds)
                g = oracle.head_chunked_bwd(x["q"], x["k"], x["v"], x["do"], w.scale, bounds, o,
                                            lse)
            else:
                o, lse = oracle.head_fwd(x["q"], x["k"], x["v"], w.scale)
                g = oracle.head_bwd(x["q"], x["k"], x["v"], x["do"], w.scale)
            per.append(time.perf_counter() - t0)
        times.append(per)
        t_work += float(np.median(per))
        heads += 1
        if outs is not None:
            got = _gpu_head(w, outs, b, h)
            for name, ref in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, *g)):
                dif = got[name] - ref
                err["max_abs"][name] = max(err["max_abs"].get(name, 0.0), float(np.abs(dif).max()))
                err["max_ref"][name] = max(err["max_ref"].get(name, 0.0), float(np.abs(ref).max()))
                err["sq_diff"][name] = err["sq_diff"].get(name, 0.0) + float((dif * dif).sum())
                err["sq_ref"][name] = err["sq_ref"].get(name, 0.0) + float((ref * ref).sum())
    if repeats > 1:
        t_work = float(np.median([sum(t[i] for t in times) for i in range(repeats)]))
    cpu_model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out = {"value": round(flops / t_work / 1e12, 6), "unit": "TFLOP/s",
           "cores": threads, "kind": "oracle",
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
           "numpy": __import__("numpy").__version__,
           "seconds": round(t_work, 3),
           "sample": f"{heads} of {len(order)} heads " +
                     ("(sequence, head)" if is_packed(w) else "(b, h)") +
                     f" of {w.name}, fwd+bwd in fp64 NumPy, {t_work:.2f} s" +
                     (f" (median of {repeats} timings)" if repeats > 1 else "")}
    errors = None
    if outs is not None:
        sq = err["sq_ref"]
        if w.dtype == "f32":
            errors = {f"{n}_rel_inf": err["max_abs"][n] / max(err["max_ref"][n], 1e-300)
                      for n in ("o", "lse", "dq", "dk", "dv")}
        else:
            errors = {"o_max_abs": err["max_abs"]["o"], "lse_max_abs": err["max_abs"]["lse"],
                      **{f"{n}_rel_fro": (err["sq_diff"][n] / sq[n]) ** 0.5 if sq[n] else 0.0
                         for n in ("dq", "dk", "dv")}}
        errors = {k: float(f"{v:.3e}") for k, v in errors.items()}
        errors["heads"] = heads
    return out, errors


def run_workload(w, steps, warmup):
    """Time `steps` steps of workload w (after `warmup` untimed ones) and
    return its bench line (without the CPU baseline)."""
    import torch
    import exact_block_wise_amd as ebw
    from exact_block_wise_amd import synth
    packed = is_packed(w)
    dev = upload(w, torch)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    tdt = q.dtype
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    o = torch.empty_like(q)
    if packed:
        cu, mx = dev["cu"], max(w.lens)
        lse = torch.empty((w.H, w.tokens), dtype=torch.float32, device="cuda")
        ws = torch.empty(ebw.bwd_varlen_workspace_bytes(q, k, cu, cu, mx, mx) // 4,
                         dtype=torch.float32, device="cuda")
    else:
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        ws = torch.empty(ebw.bwd_workspace_bytes(q, k) // 4, dtype=torch.float32, device="cuda")
    if w.chunks > 1:
        o_parts = torch.empty((w.chunks, w.B, w.H, w.Nq, w.d), dtype=torch.float32, device="cuda")
        lse_parts = torch.empty((w.chunks, w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

    # The step, as single-kernel library calls (HIP events between the calls
    # therefore time one kernel each).  Credited flops per call, in units of
    # B*H*Nq*Nkv*d: forward 4; dK/dV 8 (S, dP, dV, dK); dQ 2 (dQ; its S and
    # dP recomputation, 4 more, is extra work and not credited).  The bf16
    # dQ call runs first and also forms D = rowsum(dO * O) into the
    # workspace, which the dK/dV call then reads (the fp32 path runs the
    # preprocess inside the dQ call instead).
    calls = []
    short = is_short(w)
    if packed:
        calls.append(("fwd", 4.0, 4.0, lambda: ebw.fwd_varlen(
            q, k, v, cu, cu, mx, mx, scale=w.scale, out=o, lse=lse)))
        calls.append(("bwd_dq", 2.0, 6.0, lambda: ebw.bwd_varlen(
            q, k, v, o, do, lse, cu, cu, mx, mx, scale=w.scale, dq=dq, workspace=ws,
            need_dkdv=False)))
        calls.append(("bwd_dkdv", 8.0, 8.0, lambda: ebw.bwd_varlen(
            q, k, v, None, do, lse, cu, cu, mx, mx, scale=w.scale, dk=dk, dv=dv, workspace=ws,
            d_precomputed=True, need_dq=False)))
    elif w.chunks > 1:
        calls.append(("fwd_chunked", 4.0, 4.0, lambda: ebw.fwd_chunked(
            q, k, v, w.chunks, scale=w.scale, o_parts=o_parts, lse_parts=lse_parts)))
        calls.append(("lse_merge", 0.0, 0.0,
                      lambda: ebw.lse_merge(o_parts, lse_parts, out=o, lse=lse)))
    else:
        calls.append(("fwd", 4.0, 4.0,
                      lambda: ebw.fwd(q, k, v, scale=w.scale, out=o, lse=lse)))
    if packed:
        pass
    elif short:
        # one backward call (the packed-tile kernel forms D, dQ, dK and dV in
        # one pass; its seven products are 14 units, 10 credited)
        calls.append(("bwd", 10.0, 14.0, lambda: ebw.bwd(
            q, k, v, o, do, lse, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)))
    else:
        calls.append(("bwd_dq", 2.0, 6.0, lambda: ebw.bwd(
            q, k, v, o, do, lse, scale=w.scale, dq=dq, workspace=ws, need_dkdv=False)))
        calls.append(("bwd_dkdv", 8.0, 8.0, lambda: ebw.bwd(
            q, k, v, None, do, lse, scale=w.scale, dk=dk, dv=dv, workspace=ws,
            d_precomputed=True, need_dq=False)))

    for _ in range(warmup):
        for c in calls:
            c[3]()
    torch.cuda.synchronize()

    K = steps
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
    step_ms = sorted(ev[i][0].elapsed_time(ev[i][n]) for i in range(K))
    step_stats = {"median": round(float(np.median(step_ms)), 5), "min": round(step_ms[0], 5),
                  "p90": round(float(np.percentile(step_ms, 90)), 5)}

    u = float(w.units)
    flops = 14.0 * u
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    fwd_ms = sum(per_call[c[0]] for c in calls if c[0] in ("fwd", "fwd_chunked", "lse_merge"))
    bwd_ms = ms - fwd_ms
    # Algorithmic bytes of each call (compulsory HBM traffic: every input read
    # once, every output written once; partials, re-reads and padding are
    # overhead).  The roofline that bounds the dominant call follows from its
    # arithmetic intensity against the ridge point peak / HBM bandwidth.
    bpe = 2 if w.dtype == "bf16" else 4
    q_rows = w.tokens * w.H if packed else w.B * w.H * w.Nq      # query rows (all heads)
    kv_rows = w.tokens * w.H if packed else w.B * w.H * w.Nkv
    kv_bytes = 2 * kv_rows * w.d * bpe               # K and V (or dK and dV)
    q_bytes = q_rows * w.d * bpe                     # one query-side tensor
    row_bytes = q_rows * 4                           # one fp32 per query row
    alg_table = {
        "fwd": kv_bytes + 2 * q_bytes + row_bytes,                     # Q,K,V -> O, LSE
        "fwd_chunked": kv_bytes + q_bytes,                             # Q, K, V read
        "bwd_dq": kv_bytes + 4 * q_bytes + 2 * row_bytes,              # Q,K,V,dO,O,LSE -> dQ, D
        "bwd_dkdv": 2 * kv_bytes + 2 * q_bytes + 2 * row_bytes,        # Q,K,V,dO,LSE,D -> dK,dV
        "bwd": 2 * kv_bytes + 4 * q_bytes + 2 * row_bytes,             # ... -> dQ, dK, dV, D
    }
    kernels = {}
    for name, credit, executed, _ in calls:
        t = per_call[name]
        kernels[name] = {"ms": round(t, 5)}
        if credit:
            kernels[name]["tflops"] = round(credit * u / (t * 1e-3) / 1e12, 3)
            kernels[name]["executed_tflops"] = round(executed * u / (t * 1e-3) / 1e12, 3)
            kernels[name]["algorithmic_gbs"] = round(alg_table[name] / (t * 1e-3) / 1e9, 1)
    dom = max((c for c in calls if c[1] > 0), key=lambda c: per_call[c[0]])
    dom_t = per_call[dom[0]]
    alg_bytes = alg_table[dom[0]]
    intensity = dom[1] * u / alg_bytes
    if intensity < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = alg_bytes / (dom_t * 1e-3) / 1e9
        roof = {"kernel": dom[0], "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dom[0], w.name, short),
                "algorithmic_bytes": alg_bytes, "flop_per_byte": round(intensity, 1)}
    else:
        # bf16 products run on the matrix cores; the fp32 path is plain
        # vector FMAs (bound "alu", against the published fp32 vector peak)
        achieved = dom[1] * u / (dom_t * 1e-3) / 1e12
        roof = {"kernel": dom[0], "bound": "mfma" if w.dtype == "bf16" else "alu",
                "achieved": round(achieved, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom[0], w.name, short),
                "algorithmic_bytes": alg_bytes, "flop_per_byte": round(intensity, 1)}

    line = {
        "metric": "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak, video ViT-B N=1568",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "step_ms_stats": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) per head, rounded to the compute dtype",
        "config": ({"workload": w.name, "H": w.H, "d": w.d, "sequences": len(w.lens),
                    "tokens": w.tokens, "lengths": "x".join(map(str, sorted(set(w.lens)))) +
                    f" (each x{len(w.lens) // len(set(w.lens))})", "scale": w.scale}
                   if packed else
                   {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nkv": w.Nkv, "d": w.d,
                    "kv_chunks": w.chunks, "scale": w.scale}),
        "pct_of_peak": round(100.0 * value / peak, 2),
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "kernels": kernels,
        "roofline": roof,
    }
    return line, {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


# every workload of the default run, the headline first
ALL_WORKLOADS = ["vit_b", "vit_l", "vit_h14", "xattn", "vit_b_temporal", "vit_b_spatial",
                 "vit_b_packed", "tiny_f32"]


def summary(line):
    r = line["roofline"]
    out = {"value": line["value"], "unit": line["unit"], "pct_of_peak": line["pct_of_peak"],
           "ms_per_step": line["ms_per_step"], "step_ms_stats": line["step_ms_stats"],
           "steps": line["steps"], "warmup": line["warmup"], "dtype": line["dtype"],
           "config": line["config"],
           "roofline": {k: r[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac",
                                          "traffic", "algorithmic_bytes") if k in r}}
    for k in ("cpu_baseline", "oracle_errors"):
        if k in line:
            out[k] = line[k]
    return out


def add_oracle_leg(line, w, outs, budget_s, repeats=1):
    """The CPU oracle baseline and the GPU's errors against it on the same
    heads, both computed after the timed region."""
    import torch
    torch.cuda.synchronize()
    line["cpu_baseline"], line["oracle_errors"] = cpu_baseline(w, budget_s, outs, repeats)


def progress(msg):
    """A progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.make_mfma_profile:
        make_mfma_profile(args.make_mfma_profile, args.workload or ALL_WORKLOADS[0])
        return
    if args.make_traffic_profile:
        make_traffic_profile(args.make_traffic_profile, args.workload or ALL_WORKLOADS[0])
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import exact_block_wise_amd as ebw
    ebw.load()  # fails loudly without the built library

    w = find_workload(args.workload or ALL_WORKLOADS[0])
    line, outs = run_workload(w, args.steps, args.warmup)
    progress(f"{w.name}: {line['ms_per_step']:.4f} ms per step, {line['value']:.1f} TFLOP/s")
    if not args.no_cpu_baseline:
        add_oracle_leg(line, w, outs, args.cpu_seconds, 3 if w.name == "tiny_f32" else 1)
        progress(f"{w.name}: oracle leg {line['oracle_errors']}")
    del outs
    if args.workload is None:
        # the default run also measures every other workload (20 steps each),
        # each summarised in one entry with its own oracle baseline and
        # errors; a failure there is reported, not fatal
        others = {}
        for name in ALL_WORKLOADS[1:]:
            # the latency-bound fp32 case gets more repetitions (50 warm-up, 200 timed)
            steps, warm = (200, 50) if name == "tiny_f32" else (20, 5)
            try:
                wo = find_workload(name)
                lo, outs = run_workload(wo, steps, warm)
                progress(f"{name}: {lo['ms_per_step']:.4f} ms per step, {lo['value']:.2f} TFLOP/s")
                if not args.no_cpu_baseline:
                    add_oracle_leg(lo, wo, outs, args.other_cpu_seconds,
                                   3 if name == "tiny_f32" else 1)
                    progress(f"{name}: oracle leg {lo['oracle_errors']}")
                del outs
                others[name] = summary(lo)
            except Exception as e:  # noqa: BLE001 - reported in the line
                others[name] = {"error": f"{type(e).__name__}: {e}"[:300]}
            torch.cuda.empty_cache()
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

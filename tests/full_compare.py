"""Every head of a full-size workload against the fp64 oracle.

The GPU outputs (copied to the host) are compared head by head, element by
element, with the oracle's stacked definition (oracle.stack_fwd /
stack_bwd), run on chunks of heads in a thread pool (NumPy releases the GIL
in its array loops; each worker's BLAS is held to one thread).  The oracle
never sees GPU values: it recomputes every head from the same seeded
inputs that were uploaded.

Tolerances: bf16 O max abs 2e-2, LSE max abs 1e-3, dQ / dK / dV relative
Frobenius error 1e-2 per tensor (also checked per head); fp32: infinity-norm
relative error 1e-5 per tensor.
"""
from __future__ import annotations

import math
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from gpu_util import TOL_F32_REL, TOL_GRAD_FRO, TOL_LSE_ABS, TOL_O_ABS

GRADS = ("dq", "dk", "dv")


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class Errors:
    """Error statistics of one set of outputs, accumulated over heads."""

    def __init__(self):
        self.max_abs = {}    # tensor -> max |x - y|
        self.max_ref = {}    # tensor -> max |y|
        self.sq_diff = {}    # tensor -> sum (x - y)^2
        self.sq_ref = {}     # tensor -> sum y^2
        self.head_fro = {}   # tensor -> worst per-head relative Frobenius error
        self.heads = 0

    def add(self, name, x, y, per_head_axes):
        x = np.asarray(x, np.float64)
        y = np.asarray(y, np.float64)
        assert x.shape == y.shape, (name, x.shape, y.shape)
        assert np.all(np.isfinite(x)), f"{name}: non-finite GPU values"
        d = x - y
        self.max_abs[name] = max(self.max_abs.get(name, 0.0), float(np.abs(d).max(initial=0.0)))
        self.max_ref[name] = max(self.max_ref.get(name, 0.0), float(np.abs(y).max(initial=0.0)))
        dd = (d * d).sum(axis=per_head_axes)
        yy = (y * y).sum(axis=per_head_axes)
        self.sq_diff[name] = self.sq_diff.get(name, 0.0) + float(dd.sum())
        self.sq_ref[name] = self.sq_ref.get(name, 0.0) + float(yy.sum())
        nz = yy > 0
        worst = float(np.sqrt(dd[nz] / yy[nz]).max(initial=0.0))
        self.head_fro[name] = max(self.head_fro.get(name, 0.0), worst)

    def merge(self, other):
        for name in other.max_abs:
            self.max_abs[name] = max(self.max_abs.get(name, 0.0), other.max_abs[name])
            self.max_ref[name] = max(self.max_ref.get(name, 0.0), other.max_ref[name])
            self.sq_diff[name] = self.sq_diff.get(name, 0.0) + other.sq_diff[name]
            self.sq_ref[name] = self.sq_ref.get(name, 0.0) + other.sq_ref[name]
            self.head_fro[name] = max(self.head_fro.get(name, 0.0), other.head_fro[name])
        self.heads += other.heads

    def rel_fro(self, name):
        return math.sqrt(self.sq_diff[name] / self.sq_ref[name]) if self.sq_ref[name] else 0.0

    def rel_inf(self, name):
        return self.max_abs[name] / self.max_ref[name] if self.max_ref[name] else 0.0

    def summary(self, dtype):
        if dtype == "f32":
            return {n: self.rel_inf(n) for n in ("o", "lse", *GRADS)}
        out = {"o_max_abs": self.max_abs["o"], "lse_max_abs": self.max_abs["lse"]}
        for n in GRADS:
            out[f"{n}_rel_fro"] = self.rel_fro(n)
            out[f"{n}_worst_head_rel_fro"] = self.head_fro[n]
        return out

    def check(self, dtype, what):
        """Assert the stated tolerances; returns the summary."""
        s = self.summary(dtype)
        if dtype == "f32":
            bad = {k: v for k, v in s.items() if v > TOL_F32_REL}
        else:
            bad = {}
            if s["o_max_abs"] > TOL_O_ABS:
                bad["o_max_abs"] = s["o_max_abs"]
            if s["lse_max_abs"] > TOL_LSE_ABS:
                bad["lse_max_abs"] = s["lse_max_abs"]
            for n in GRADS:
                for key in (f"{n}_rel_fro", f"{n}_worst_head_rel_fro"):
                    if s[key] > TOL_GRAD_FRO:
                        bad[key] = s[key]
        assert not bad, f"{what}: over tolerance {bad}"
        return s


def _host(t):
    """GPU tensor -> host torch tensor of the same dtype (one copy)."""
    return t.detach().to("cpu")


def _f64(t):
    return t.float().numpy().astype(np.float64)


def _run_chunks(chunks, fn, threads):
    from threadpoolctl import threadpool_limits
    total = Errors()
    with threadpool_limits(1):
        with ThreadPoolExecutor(threads) as ex:
            for part in ex.map(fn, chunks):
                total.merge(part)
    return total


def compare_dense(inputs, outputs, scale, dtype, say=print, threads=None):
    """inputs: host float32 arrays q [B,H,Nq,d], k, v [B,H,Nkv,d], do.
    outputs: {label: {"o", "lse", "dq", "dk", "dv": GPU tensors}}, every set
    compared with the same oracle values.  Returns {label: Errors}."""
    q, k, v, do = (inputs[n] for n in ("q", "k", "v", "do"))
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    n_heads = B * H
    threads = threads or _threads()
    host = {lab: {n: _host(t) for n, t in outs.items()} for lab, outs in outputs.items()}
    flat = lambda a: a.reshape(n_heads, *a.shape[2:])
    qf, kf, vf, dof = map(flat, (q, k, v, do))
    hf = {lab: {n: t.reshape(n_heads, *t.shape[2:]) for n, t in o.items()}
          for lab, o in host.items()}
    # heads per chunk: about 8M scores per chunk, and at least 4 chunks per thread
    per = max(1, min(8_000_000 // max(1, Nq * Nkv), -(-n_heads // (4 * threads))))
    chunks = [(i, min(i + per, n_heads)) for i in range(0, n_heads, per)]

    def work(ch):
        lo, hi = ch
        o_ref, lse_ref = oracle.stack_fwd(qf[lo:hi], kf[lo:hi], vf[lo:hi], scale)
        g_ref = oracle.stack_bwd(qf[lo:hi], kf[lo:hi], vf[lo:hi], dof[lo:hi], scale)
        res = {}
        for lab, o in hf.items():
            e = Errors()
            e.heads = hi - lo
            e.add("o", _f64(o["o"][lo:hi]), o_ref, (1, 2))
            e.add("lse", _f64(o["lse"][lo:hi]), lse_ref, (1,))
            for n, r in zip(GRADS, g_ref):
                e.add(n, _f64(o[n][lo:hi]), r, (1, 2))
            res[lab] = e
        return res

    from threadpoolctl import threadpool_limits
    t0 = time.perf_counter()
    totals = {lab: Errors() for lab in outputs}
    with threadpool_limits(1):
        with ThreadPoolExecutor(threads) as ex:
            for part in ex.map(work, chunks):
                for lab, e in part.items():
                    totals[lab].merge(e)
    say(f"  oracle over {n_heads} heads in {len(chunks)} chunks, {threads} threads: "
        f"{time.perf_counter() - t0:.1f} s")
    return totals


def compare_packed(w, inputs, outputs, say=print, threads=None):
    """Packed sequences: inputs are host [T,H,d] float32 arrays (q, k, v,
    do), outputs GPU tensors o, dq, dk, dv [T,H,d] and lse [H,T].  Each
    (sequence, head) is one oracle head; sequences of equal length are
    stacked."""
    threads = threads or _threads()
    host = {n: _host(t) for n, t in outputs.items()}
    cu = w.cu
    by_len = {}
    for s, n in enumerate(w.lens):
        by_len.setdefault(n, []).append(s)
    jobs = []
    for n, seqs in by_len.items():
        per = max(1, 8_000_000 // max(1, n * n))
        pairs = [(s, h) for s in seqs for h in range(w.H)]
        for i in range(0, len(pairs), per):
            jobs.append((n, pairs[i:i + per]))

    def rows(a, s, h):
        return a[cu[s]:cu[s + 1], h]

    def work(job):
        n, pairs = job
        x = {t: np.stack([rows(inputs[t], s, h) for s, h in pairs]) for t in ("q", "k", "v", "do")}
        o_ref, lse_ref = oracle.stack_fwd(x["q"], x["k"], x["v"], w.scale)
        g_ref = oracle.stack_bwd(x["q"], x["k"], x["v"], x["do"], w.scale)
        e = Errors()
        e.heads = len(pairs)
        e.add("o", np.stack([_f64(rows(host["o"], s, h)) for s, h in pairs]), o_ref, (1, 2))
        e.add("lse", np.stack([_f64(host["lse"][h, cu[s]:cu[s + 1]]) for s, h in pairs]),
              lse_ref, (1,))
        for nm, r in zip(GRADS, g_ref):
            e.add(nm, np.stack([_f64(rows(host[nm], s, h)) for s, h in pairs]), r, (1, 2))
        return e

    t0 = time.perf_counter()
    total = _run_chunks(jobs, work, threads)
    say(f"  oracle over {total.heads} (sequence, head) problems, {threads} threads: "
        f"{time.perf_counter() - t0:.1f} s")
    return total


# one line per compared workload, printed again in pytest's terminal summary
# (tests/conftest.py) so that a quiet run's log still records the errors
REPORT = []


def log_errors(say, what, errs, dtype):
    s = errs.summary(dtype)
    line = f"{what}: " + ", ".join(f"{k} {v:.3e}" for k, v in s.items())
    REPORT.append(line)
    say("  " + line)

"""Checks that pin the oracle to facts outside itself.

Each check takes the function under test as an argument and returns the
largest violation it found (0 for a perfect match, inf for a crash or a shape
mismatch), so the same checks serve the oracle's own tests and the mutation
test that plants mistakes in copies of it.

Sources of truth: pure-Python brute force, closed forms, central finite
differences, torch autograd in fp64, and invariants of the mathematics.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _safe(fn):
    def wrapped(*a, **kw):
        try:
            with np.errstate(all="ignore"):
                r = fn(*a, **kw)
            return float(r) if np.isfinite(r) else math.inf
        except (ValueError, IndexError, TypeError, FloatingPointError):
            return math.inf
    wrapped.__name__ = fn.__name__
    return wrapped


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _expr(s):
    return float(eval(s, {"__builtins__": {}}, {"e": math.e, "ln": math.log}))


def _maxdiff(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return math.inf
    return float(np.max(np.abs(a - b))) if a.size else 0.0


# ----------------------------------------------------------------- forward

@_safe
def fwd_vs_brute(head_fwd, brute_fwd, n_cases=20):
    """Tiny random heads (N <= 8, d <= 4) against pure-Python loops."""
    worst = 0.0
    for seed in range(n_cases):
        g = _rng(seed)
        nq, nkv, d = int(g.integers(1, 9)), int(g.integers(1, 9)), int(g.integers(1, 5))
        q, k, v = (g.standard_normal((n, d)) for n in (nq, nkv, nkv))
        scale = float(g.uniform(0.2, 1.5))
        o, lse = head_fwd(q, k, v, scale)
        ob, lb = brute_fwd(q.tolist(), k.tolist(), v.tolist(), scale)
        worst = max(worst, _maxdiff(o, ob), _maxdiff(lse, lb))
    return worst


@_safe
def fwd_golden(head_fwd):
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    worst = 0.0
    for c in cases:
        o, lse = head_fwd(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"])
        eo = [[_expr(x) for x in row] for row in c["o"]]
        el = [_expr(x) for x in c["lse"]]
        worst = max(worst, _maxdiff(o, eo), _maxdiff(lse, el))
    return worst


@_safe
def fwd_closed_forms(head_fwd):
    g = _rng(101)
    worst = 0.0
    nq, nkv, d, scale = 5, 7, 3, 0.6
    q, k, v = g.standard_normal((nq, d)), g.standard_normal((nkv, d)), g.standard_normal((nkv, d))
    # Q = 0: uniform weights, O = mean of V rows, LSE = ln Nkv
    o, lse = head_fwd(np.zeros((nq, d)), k, v, scale)
    worst = max(worst, _maxdiff(o, np.tile(v.mean(0), (nq, 1))),
                _maxdiff(lse, np.full(nq, math.log(nkv))))
    # Nkv = 1: O = v_1, LSE = scale q.k_1
    o, lse = head_fwd(q, k[:1], v[:1], scale)
    worst = max(worst, _maxdiff(o, np.tile(v[0], (nq, 1))),
                _maxdiff(lse, scale * (q @ k[0])))
    # all keys equal: uniform weights
    kk = np.tile(k[0], (nkv, 1))
    o, lse = head_fwd(q, kk, v, scale)
    worst = max(worst, _maxdiff(o, np.tile(v.mean(0), (nq, 1))),
                _maxdiff(lse, scale * (q @ k[0]) + math.log(nkv)))
    # V columns constant: O is that constant
    cv = np.tile(np.array([1.5, -2.0, 0.25]), (nkv, 1))
    o, _ = head_fwd(q, k, cv, scale)
    worst = max(worst, _maxdiff(o, np.tile(cv[0], (nq, 1))))
    # V = I (Nkv = d): O = P, rows sum to 1, and P_ij = exp(S_ij - LSE_i)
    kd = g.standard_normal((d, d))
    o, lse = head_fwd(q, kd, np.eye(d), scale)
    p_expected = np.array([[math.exp(scale * float(q[i] @ kd[j]) - lse[i]) for j in range(d)]
                           for i in range(nq)])
    worst = max(worst, _maxdiff(o.sum(1), np.ones(nq)), _maxdiff(o, p_expected))
    return worst


@_safe
def fwd_invariants(head_fwd):
    g = _rng(202)
    nq, nkv, d, scale = 6, 9, 4, 0.5
    q, k, v = g.standard_normal((nq, d)), g.standard_normal((nkv, d)), g.standard_normal((nkv, d))
    o, lse = head_fwd(q, k, v, scale)
    worst = 0.0
    # permuting key/value rows together changes nothing
    perm = g.permutation(nkv)
    o2, l2 = head_fwd(q, k[perm], v[perm], scale)
    worst = max(worst, _maxdiff(o, o2), _maxdiff(lse, l2))
    # permuting query rows permutes the outputs
    pq = g.permutation(nq)
    o3, l3 = head_fwd(q[pq], k, v, scale)
    worst = max(worst, _maxdiff(o[pq], o3), _maxdiff(lse[pq], l3))
    # shifting every key by u leaves O and adds scale q_i.u to LSE_i
    u = g.standard_normal(d)
    o4, l4 = head_fwd(q, k + u, v, scale)
    worst = max(worst, _maxdiff(o, o4), _maxdiff(lse + scale * (q @ u), l4))
    # max_j S_ij <= LSE_i <= max_j S_ij + ln Nkv
    smax = (scale * (q @ k.T)).max(1)
    viol = np.maximum(smax - lse, 0) + np.maximum(lse - smax - math.log(nkv), 0)
    worst = max(worst, float(viol.max()))
    # a peaky softmax (scores ~ 60) stays finite and still sums to one
    o5, l5 = head_fwd(q * 40, k, np.eye(d)[:nkv] if nkv <= d else np.vstack([np.eye(d)] * 3)[:nkv], scale)
    worst = max(worst, 0.0 if np.all(np.isfinite(o5)) and np.all(np.isfinite(l5)) else math.inf)
    return worst


# ----------------------------------------------------------------- backward

def _loss(head_fwd, q, k, v, do, scale):
    o, _ = head_fwd(q, k, v, scale)
    return float((np.asarray(o) * do).sum())


@_safe
def bwd_finite_differences(head_fwd, head_bwd, seeds=(0, 1, 2), h=1e-6):
    """Relative error of (dQ, dK, dV) against central differences of
    L = sum(dO * O), with O from the forward under test."""
    worst = 0.0
    for seed in seeds:
        g = _rng(1000 + seed)
        nq, nkv, d = 3 + seed, 4 + 2 * seed, 2 + seed
        scale = 0.8
        q, k, v, do = (g.standard_normal(s) for s in ((nq, d), (nkv, d), (nkv, d), (nq, d)))
        grads = head_bwd(q, k, v, do, scale)
        args = [q, k, v]
        for which in range(3):
            x = args[which]
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                ap, am = list(args), list(args)
                ap[which], am[which] = xp, xm
                num[idx] = (_loss(head_fwd, *ap, do, scale) - _loss(head_fwd, *am, do, scale)) / (2 * h)
            gr = np.asarray(grads[which])
            if gr.shape != num.shape:
                return math.inf
            worst = max(worst, float(np.abs(gr - num).max() / max(np.abs(num).max(), 1e-300)))
    return worst


@_safe
def bwd_vs_autograd(head_bwd, seeds=(0, 1, 2, 3)):
    """The definition differentiated by torch autograd in fp64 on the CPU."""
    import torch
    worst = 0.0
    for seed in seeds:
        g = _rng(2000 + seed)
        nq, nkv, d = 5 + seed, 11 - seed, 3 + seed % 2
        scale = 0.45
        arrs = [g.standard_normal(s) for s in ((nq, d), (nkv, d), (nkv, d), (nq, d))]
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in arrs[:3])
        o = torch.softmax(scale * tq @ tk.T, dim=-1) @ tv
        o.backward(torch.tensor(arrs[3], dtype=torch.float64))
        got = head_bwd(*arrs, scale)
        for a, t in zip(got, (tq, tk, tv)):
            worst = max(worst, _maxdiff(a, t.grad.numpy()))
    return worst


@_safe
def bwd_golden(head_bwd):
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["backward_cases"]
    worst = 0.0
    for c in cases:
        got = head_bwd(*(np.array(c[n]) for n in ("q", "k", "v", "do")), c["scale"])
        for a, name in zip(got, ("dq", "dk", "dv")):
            worst = max(worst, _maxdiff(a, [[_expr(x) for x in row] for row in c[name]]))
    return worst


@_safe
def bwd_invariants(head_bwd):
    g = _rng(303)
    nq, nkv, d, scale = 7, 10, 4, 0.55
    q, k, v, do = (g.standard_normal(s) for s in ((nq, d), (nkv, d), (nkv, d), (nq, d)))
    dq, dk, dv = head_bwd(q, k, v, do, scale)
    worst = 0.0
    # rows of dS sum to zero, hence sum_j dK_j = 0
    worst = max(worst, float(np.abs(np.asarray(dk).sum(0)).max()))
    # rows of P sum to one, hence sum_j dV_j = sum_i dO_i
    worst = max(worst, _maxdiff(np.asarray(dv).sum(0), do.sum(0)))
    # key/value permutation permutes dK and dV and leaves dQ
    perm = g.permutation(nkv)
    dq2, dk2, dv2 = head_bwd(q, k[perm], v[perm], do, scale)
    worst = max(worst, _maxdiff(dq, dq2), _maxdiff(np.asarray(dk)[perm], dk2),
                _maxdiff(np.asarray(dv)[perm], dv2))
    return worst


# ----------------------------------------------------------------- merge

@_safe
def merge_any_split(head_fwd, lse_merge, seeds=range(12)):
    """The merge of any split of the keys equals the unsplit result."""
    worst = 0.0
    for seed in seeds:
        g = _rng(4000 + seed)
        nq, nkv, d, scale = int(g.integers(1, 6)), int(g.integers(2, 40)), 3, 0.7
        q, k, v = g.standard_normal((nq, d)), g.standard_normal((nkv, d)), g.standard_normal((nkv, d))
        o, lse = head_fwd(q, k, v, scale)
        perm = g.permutation(nkv)
        n_parts = int(g.integers(1, 7))
        cuts = np.sort(g.integers(0, nkv + 1, size=n_parts - 1))   # empty chunks allowed
        bounds = [0, *cuts.tolist(), nkv]
        parts = []
        for c in range(n_parts):
            idx = perm[bounds[c]:bounds[c + 1]]
            parts.append(head_fwd(q, k[idx], v[idx], scale))
        order = g.permutation(n_parts)
        om, lm = lse_merge(np.stack([parts[i][0] for i in order]),
                           np.stack([parts[i][1] for i in order]))
        worst = max(worst, _maxdiff(o, om), _maxdiff(lse, lm))
        # a merge tree: merge the two halves' merges
        if n_parts >= 2:
            h = n_parts // 2
            left = lse_merge(np.stack([p[0] for p in parts[:h]]), np.stack([p[1] for p in parts[:h]]))
            right = lse_merge(np.stack([p[0] for p in parts[h:]]), np.stack([p[1] for p in parts[h:]]))
            ot, lt = lse_merge(np.stack([left[0], right[0]]), np.stack([left[1], right[1]]))
            worst = max(worst, _maxdiff(o, ot), _maxdiff(lse, lt))
    return worst


@_safe
def merge_empty_parts(lse_merge):
    """-inf partials get weight 0; an all-empty row is O = 0, LSE = -inf."""
    o_parts = np.array([[[1.0, 2.0]], [[5.0, 7.0]], [[9.0, 9.0]]])
    lse_parts = np.array([[math.log(2.0)], [-math.inf], [math.log(6.0)]])
    o, lse = lse_merge(o_parts, lse_parts)
    worst = max(_maxdiff(lse, [math.log(8.0)]),
                _maxdiff(o, [[(2 * 1 + 6 * 9) / 8, (2 * 2 + 6 * 9) / 8]]))
    o, lse = lse_merge(o_parts[:2] * 0 + 3.0, np.full((2, 1), -math.inf))
    if not (np.all(o == 0.0) and np.all(np.isneginf(lse))):
        return math.inf
    return worst


@_safe
def chunked_bwd_vs_unsplit(head_bwd, head_chunked_fwd, head_chunked_bwd, seeds=range(6)):
    worst = 0.0
    for seed in seeds:
        g = _rng(5000 + seed)
        nq, nkv, d, scale = int(g.integers(1, 7)), int(g.integers(3, 30)), 3, 0.6
        q, k, v, do = (g.standard_normal(s) for s in ((nq, d), (nkv, d), (nkv, d), (nq, d)))
        cuts = np.sort(g.integers(0, nkv + 1, size=int(g.integers(1, 5))))
        bounds = [0, *cuts.tolist(), nkv]
        o, lse, _, _ = head_chunked_fwd(q, k, v, scale, bounds)
        got = head_chunked_bwd(q, k, v, do, scale, bounds, o, lse)
        ref = head_bwd(q, k, v, do, scale)
        for a, b in zip(got, ref):
            worst = max(worst, _maxdiff(a, b))
    return worst


# ----------------------------------------------------------------- stacks

@_safe
def stack_vs_brute(stack_fwd, brute_fwd, n_cases=8):
    """Stacks of 1-5 tiny random heads: every head against pure-Python loops
    over its own rows only."""
    worst = 0.0
    for seed in range(n_cases):
        g = _rng(100 + seed)
        n = int(g.integers(1, 6))
        nq, nkv, d = int(g.integers(1, 7)), int(g.integers(1, 7)), int(g.integers(1, 5))
        q, k, v = (g.standard_normal((n, m, d)) for m in (nq, nkv, nkv))
        scale = float(g.uniform(0.2, 1.5))
        o, lse = stack_fwd(q, k, v, scale)
        for i in range(n):
            ob, lb = brute_fwd(q[i].tolist(), k[i].tolist(), v[i].tolist(), scale)
            worst = max(worst, _maxdiff(o[i], ob), _maxdiff(lse[i], lb))
    return worst


@_safe
def stack_bwd_vs_autograd(stack_bwd, seeds=(0, 1, 2)):
    """Gradients of a stack of heads against torch autograd (fp64, CPU) of
    the naive definition, summed loss over all heads."""
    import torch
    worst = 0.0
    for seed in seeds:
        g = _rng(200 + seed)
        n, nq, nkv, d = 3, int(g.integers(1, 6)), int(g.integers(1, 6)), int(g.integers(1, 5))
        q, k, v, do = (g.standard_normal((n, m, d)) for m in (nq, nkv, nkv, nq))
        scale = float(g.uniform(0.3, 1.2))
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        o = torch.softmax(scale * tq @ tk.transpose(1, 2), dim=2) @ tv
        (o * torch.tensor(do)).sum().backward()
        got = stack_bwd(q, k, v, do, scale)
        for x, t in zip(got, (tq, tk, tv)):
            worst = max(worst, _maxdiff(x, t.grad.numpy()))
    return worst

"""Plain, slow fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The product
(the HIP library and its Python binding) never calls it and shares no code
with it.

What it computes, and the passages it follows:

* Attention is a weighted average of the value rows whose weights come from
  query-key dot products passed through a softmax ("Training a Large Video
  Model on a Single Machine in a Day", §3, "Flash Attention" paragraph, which
  cites Vaswani et al. 2017).  With the scale inside the softmax:
      S = scale * Q K^T,  P = softmax_rows(S),  O = P V.
* The block-wise method of that page (§1 and §3: results of SRAM-sized blocks
  are combined into the final output, the N x N weights are never stored) and
  the distributed cross-attention of the LV-XAttn abstract ("exact"; the lay
  summary: the output of the model does not change) both reach this result
  exactly, so the oracle is the definition itself, materialising S and P for
  one (batch, head) at a time.
* The per-row log-sum-exp LSE_i = ln sum_j exp(S_ij) is the statistic that
  lets partial results over disjoint key/value sets be combined exactly
  (reading of the LV-XAttn abstract: key/value blocks stay where they are and
  only query-sized results move).
* Training through the method (AVION page, §4.1 and Fig. 4 measure
  forward + backward throughput) needs the gradients; the oracle uses the
  closed-form derivative of the definition, with P recomputed from LSE.

Everything is float64 on the values it is given (the bf16-rounded or fp32
inputs, and the fp32-rounded scale).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# One head: the definition
# --------------------------------------------------------------------------

def head_scores(q, k, scale):
    """S = scale * Q K^T  (Nq x Nkv)."""
    return float(scale) * (_f64(q) @ _f64(k).T)


def head_lse(s):
    """LSE_i = ln sum_j exp(S_ij), evaluated around the row maximum.

    An empty row (Nkv = 0) has LSE = -inf (the log of an empty sum).
    """
    if s.shape[1] == 0:
        return np.full(s.shape[0], -np.inf)
    m = s.max(axis=1)
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def head_fwd(q, k, v, scale):
    """(O, LSE) of one head: O = softmax(scale Q K^T) V.

    For an empty key set the output row is defined as 0 (no weights).
    """
    s = head_scores(q, k, scale)
    lse = head_lse(s)
    if s.shape[1] == 0:
        return np.zeros((s.shape[0], np.shape(v)[1])), lse
    p = np.exp(s - lse[:, None])
    return p @ _f64(v), lse


def head_bwd(q, k, v, do, scale):
    """(dQ, dK, dV) of one head for the loss L = sum(dO * O).

    Closed form of the derivative of O = softmax(S) V with S = scale Q K^T:
      dV = P^T dO
      dP = dO V^T
      D_i = sum_j P_ij dP_ij
      dS = P * (dP - D)            (softmax Jacobian applied row by row)
      dQ = scale dS K
      dK = scale dS^T Q
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    s = head_scores(q, k, scale)
    lse = head_lse(s)
    p = np.exp(s - lse[:, None])
    dv = p.T @ do
    dp = do @ v.T
    dsum = (p * dp).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


# --------------------------------------------------------------------------
# Exact combination of partial results over disjoint key/value sets
# --------------------------------------------------------------------------

def lse_merge(o_parts, lse_parts):
    """Merge C partials (O_c, LSE_c) computed over disjoint key/value sets.

    o_parts: [C, ..., Nq, d]; lse_parts: [C, ..., Nq].
    Because exp(LSE) of the union is the sum of exp(LSE_c):
      M = max_c LSE_c,  LSE = M + ln sum_c exp(LSE_c - M),
      O = sum_c exp(LSE_c - LSE) O_c.
    A partial with LSE_c = -inf (an empty chunk) gets weight 0; if every
    partial is -inf the merged row is O = 0, LSE = -inf.
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe)           # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    lse_safe = np.where(empty, 0.0, lse)
    coef = np.where(empty, 0.0, np.exp(lse_parts - lse_safe))
    o = (coef[..., None] * o_parts).sum(axis=0)
    return o, lse


def head_chunked_fwd(q, k, v, scale, bounds):
    """Forward over key/value chunks [bounds[c], bounds[c+1]) then merged.

    Returns (O, LSE, O_parts, LSE_parts).
    """
    parts_o, parts_l = [], []
    for c in range(len(bounds) - 1):
        lo, hi = bounds[c], bounds[c + 1]
        o_c, l_c = head_fwd(q, k[lo:hi], v[lo:hi], scale)
        parts_o.append(o_c)
        parts_l.append(l_c)
    o_parts, lse_parts = np.stack(parts_o), np.stack(parts_l)
    o, lse = lse_merge(o_parts, lse_parts)
    return o, lse, o_parts, lse_parts


def head_chunked_bwd(q, k, v, do, scale, bounds, o, lse):
    """Backward chunk by chunk from the merged (O, LSE).

    With the merged LSE every chunk recomputes the global softmax columns
    P_c = exp(S_c - LSE), and D_i = dO_i . O_i is the full-row value, so
    dK_c and dV_c are the chunk's rows of the unsplit gradients and dQ is
    the sum of the chunks' contributions.
    """
    q, k, v, do, o, lse = map(_f64, (q, k, v, do, o, lse))
    dsum = (do * o).sum(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c in range(len(bounds) - 1):
        lo, hi = bounds[c], bounds[c + 1]
        s = head_scores(q, k[lo:hi], scale)
        p = np.exp(s - lse[:, None])
        dv[lo:hi] = p.T @ do
        dp = do @ v[lo:hi].T
        ds = p * (dp - dsum[:, None])
        dq += float(scale) * (ds @ k[lo:hi])
        dk[lo:hi] = float(scale) * (ds.T @ q)
    return dq, dk, dv


# --------------------------------------------------------------------------
# A stack of independent heads: the same definition, one matrix product per
# head through NumPy's stacked matmul.  Used where a workload has too many
# small heads for a Python loop over head_fwd / head_bwd (divided space-time
# attention: tens of thousands of 8-token sequences).
# --------------------------------------------------------------------------

def _kt(k):
    """K^T of every head of a stack [n, N, d] -> [n, d, N]."""
    return np.swapaxes(k, -1, -2)


def stack_fwd(q, k, v, scale):
    """(O [n,Nq,d], LSE [n,Nq]) of n independent heads, q [n,Nq,d],
    k and v [n,Nkv,d]: per head S = scale Q K^T, LSE_i = ln sum_j exp(S_ij),
    O = exp(S - LSE) V.  An empty key set gives O = 0, LSE = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, nq, nkv = q.shape[0], q.shape[1], k.shape[1]
    if nkv == 0:
        return np.zeros((n, nq, v.shape[2])), np.full((n, nq), -np.inf)
    s = float(scale) * (q @ _kt(k))
    m = s.max(axis=2)
    lse = m + np.log(np.exp(s - m[:, :, None]).sum(axis=2))
    p = np.exp(s - lse[:, :, None])
    return p @ v, lse


def stack_bwd(q, k, v, do, scale):
    """(dQ, dK, dV) of n independent heads for L = sum(dO * O); the closed
    form of head_bwd applied to every head of the stack."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if k.shape[1] == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    s = float(scale) * (q @ _kt(k))
    m = s.max(axis=2)
    lse = m + np.log(np.exp(s - m[:, :, None]).sum(axis=2))
    p = np.exp(s - lse[:, :, None])
    pt = np.swapaxes(p, -1, -2)
    dv = pt @ do
    dp = do @ _kt(v)
    dsum = (p * dp).sum(axis=2)
    ds = p * (dp - dsum[:, :, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (np.swapaxes(ds, -1, -2) @ q)
    return dq, dk, dv


# --------------------------------------------------------------------------
# [B, H, N, d] wrappers: one head at a time
# --------------------------------------------------------------------------

def ref_fwd(q, k, v, scale, heads=None):
    """O [B,H,Nq,d], LSE [B,H,Nq] for all heads (or the listed (b, h))."""
    B, H, Nq, d = np.shape(q)
    o = np.zeros((B, H, Nq, np.shape(v)[3]))
    lse = np.zeros((B, H, Nq))
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        o[b, h], lse[b, h] = head_fwd(q[b, h], k[b, h], v[b, h], scale)
    return o, lse


def ref_bwd(q, k, v, do, scale, heads=None):
    """dQ, dK, dV [B,H,N,d] for all heads (or the listed (b, h))."""
    dq = np.zeros(np.shape(q))
    dk = np.zeros(np.shape(k))
    dv = np.zeros(np.shape(v))
    B, H = np.shape(q)[:2]
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        dq[b, h], dk[b, h], dv[b, h] = head_bwd(q[b, h], k[b, h], v[b, h],
                                                do[b, h], scale)
    return dq, dk, dv


def brute_fwd(q, k, v, scale):
    """Pure-Python triple loops (no NumPy arithmetic) for tiny inputs.

    q, k, v are nested lists [N][d] of floats for one head.
    """
    import math
    out, lses = [], []
    for qi in q:
        s = [float(scale) * math.fsum(a * b for a, b in zip(qi, kj)) for kj in k]
        m = max(s)
        z = math.fsum(math.exp(x - m) for x in s)
        lse = m + math.log(z)
        w = [math.exp(x - lse) for x in s]
        out.append([math.fsum(w[j] * k_row[c] for j, k_row in enumerate(v))
                    for c in range(len(v[0]))])
        lses.append(lse)
    return out, lses

"""The fp64 oracle against brute force, closed forms, finite differences,
autograd and invariants; then the same checks against planted mistakes.

CPU only.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as A
import pins

TOL = 1e-12


def test_fwd_brute_force():
    assert pins.fwd_vs_brute(A.head_fwd, A.brute_fwd) < 1e-13


def test_fwd_golden_closed_forms():
    assert pins.fwd_golden(A.head_fwd) < TOL


def test_fwd_closed_forms():
    assert pins.fwd_closed_forms(A.head_fwd) < TOL


def test_fwd_invariants():
    assert pins.fwd_invariants(A.head_fwd) < 1e-11


def test_bwd_finite_differences():
    assert pins.bwd_finite_differences(A.head_fwd, A.head_bwd) < 1e-7


def test_bwd_autograd():
    assert pins.bwd_vs_autograd(A.head_bwd) < TOL


def test_bwd_golden():
    assert pins.bwd_golden(A.head_bwd) < TOL


def test_bwd_invariants():
    assert pins.bwd_invariants(A.head_bwd) < 1e-12


def test_merge_any_split():
    assert pins.merge_any_split(A.head_fwd, A.lse_merge) < 1e-13


def test_merge_empty_parts():
    assert pins.merge_empty_parts(A.lse_merge) < 1e-14


def test_chunked_bwd_equals_unsplit():
    assert pins.chunked_bwd_vs_unsplit(A.head_bwd, A.head_chunked_fwd,
                                       A.head_chunked_bwd) < 1e-13


def test_batched_wrappers_match_heads():
    g = np.random.Generator(np.random.PCG64(9))
    q, k, v, do = (g.standard_normal((2, 3, n, 4)) for n in (5, 7, 7, 5))
    o, lse = oracle.ref_fwd(q, k, v, 0.5)
    dq, dk, dv = oracle.ref_bwd(q, k, v, do, 0.5)
    for b in range(2):
        for h in range(3):
            oh, lh = A.head_fwd(q[b, h], k[b, h], v[b, h], 0.5)
            assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h])
            gh = A.head_bwd(q[b, h], k[b, h], v[b, h], do[b, h], 0.5)
            for x, y in zip(gh, (dq, dk, dv)):
                assert np.array_equal(x, y[b, h])


# --------------------------------------------------------------------------
# The stacked functions (many independent heads in one call) carry every pin
# of the per-head ones, through one-head stacks, plus a check that heads of
# a stack never mix.
# --------------------------------------------------------------------------

def _one_head_fwd(q, k, v, scale):
    o, lse = A.stack_fwd(np.asarray(q)[None], np.asarray(k)[None], np.asarray(v)[None], scale)
    return o[0], lse[0]


def _one_head_bwd(q, k, v, do, scale):
    g = A.stack_bwd(*(np.asarray(x)[None] for x in (q, k, v, do)), scale)
    return tuple(x[0] for x in g)


def test_stack_pins():
    assert pins.fwd_vs_brute(_one_head_fwd, A.brute_fwd) < 1e-13
    assert pins.fwd_golden(_one_head_fwd) < TOL
    assert pins.fwd_closed_forms(_one_head_fwd) < TOL
    assert pins.fwd_invariants(_one_head_fwd) < 1e-11
    assert pins.bwd_finite_differences(_one_head_fwd, _one_head_bwd) < 1e-7
    assert pins.bwd_vs_autograd(_one_head_bwd) < TOL
    assert pins.bwd_golden(_one_head_bwd) < TOL
    assert pins.bwd_invariants(_one_head_bwd) < 1e-12


def test_stack_heads_stay_separate():
    assert pins.stack_vs_brute(A.stack_fwd, A.brute_fwd) < 1e-13
    assert pins.stack_bwd_vs_autograd(A.stack_bwd) < TOL
    o, lse = A.stack_fwd(np.ones((2, 3, 2)), np.zeros((2, 0, 2)), np.zeros((2, 0, 2)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _stack_fwd_heads_mixed(q, k, v, scale):
    # K^T taken over the wrong axes: head n meets the keys of other heads
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    s = float(scale) * np.einsum("nid,mjd->nij", q, k[::-1])
    lse = np.log(np.exp(s).sum(axis=2))
    return np.exp(s - lse[:, :, None]) @ v, lse


def _stack_bwd_sum_over_heads(q, k, v, do, scale):
    dq, dk, dv = A.stack_bwd(q, k, v, do, scale)
    return dq, dk, dv + dv.sum(axis=0, keepdims=True) - dv  # every head gets the total


def test_stack_pins_catch_mixed_heads():
    assert pins.stack_vs_brute(_stack_fwd_heads_mixed, A.brute_fwd) > 1e-6
    assert pins.stack_bwd_vs_autograd(_stack_bwd_sum_over_heads) > 1e-6


def test_empty_key_set():
    o, lse = A.head_fwd(np.ones((3, 2)), np.zeros((0, 2)), np.zeros((0, 2)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# Planted mistakes: every plausible slip in a copy of the oracle must fail
# at least one pin.  The copies live here, never in the oracle itself.
# --------------------------------------------------------------------------

def _fwd_no_scale(q, k, v, scale):
    return A.head_fwd(q, k, v, 1.0)


def _fwd_scale_outside(q, k, v, scale):
    o, lse = A.head_fwd(q, k, v, 1.0)
    return o, scale * lse


def _fwd_unnormalised(q, k, v, scale):
    s = A.head_scores(q, k, scale)
    lse = A.head_lse(s)
    return np.exp(s) @ v, lse


def _fwd_lse_drops_max(q, k, v, scale):
    s = A.head_scores(q, k, scale)
    m = s.max(1)
    o, _ = A.head_fwd(q, k, v, scale)
    return o, np.log(np.exp(s - m[:, None]).sum(1))


def _fwd_softmax_wrong_axis(q, k, v, scale):
    s = A.head_scores(q, k, scale)
    p = np.exp(s - s.max(0)[None, :])
    p = p / p.sum(0)[None, :]
    return p @ v, A.head_lse(s)


def _fwd_v_reversed(q, k, v, scale):
    return A.head_fwd(q, k, np.asarray(v)[::-1], scale)


def _fwd_off_by_one_key(q, k, v, scale):
    if len(k) > 1:
        return A.head_fwd(q, k[:-1], v[:-1], scale)
    return A.head_fwd(q, k, v, scale)


def _fwd_k_transposed_roles(q, k, v, scale):
    # scores taken as K Q^T then transposed back -- fine -- but V weighted by
    # the column softmax: a transposed operand
    s = A.head_scores(k, q, scale)
    lse = A.head_lse(s.T)
    p = np.exp(s - A.head_lse(s)[:, None])
    return p.T @ v if p.shape[1] == len(q) and p.shape[0] == len(v) else p @ v, lse


FWD_MUTANTS = [_fwd_no_scale, _fwd_scale_outside, _fwd_unnormalised,
               _fwd_lse_drops_max, _fwd_softmax_wrong_axis, _fwd_v_reversed,
               _fwd_off_by_one_key, _fwd_k_transposed_roles]


@pytest.mark.parametrize("mutant", FWD_MUTANTS, ids=lambda f: f.__name__)
def test_forward_pins_catch_planted_mistakes(mutant):
    errs = [pins.fwd_vs_brute(mutant, A.brute_fwd), pins.fwd_golden(mutant),
            pins.fwd_closed_forms(mutant), pins.fwd_invariants(mutant)]
    assert max(errs) > 1e-6, errs


def _bwd_parts(q, k, v, do, scale):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = A.head_scores(q, k, scale)
    p = np.exp(s - A.head_lse(s)[:, None])
    return q, k, v, do, p


def _bwd_drop_d(q, k, v, do, scale):
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    ds = p * (do @ v.T)
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_wrong_sign(q, k, v, do, scale):
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    dp = do @ v.T
    ds = p * ((p * dp).sum(1)[:, None] - dp)
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_no_scale(q, k, v, do, scale):
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(1)[:, None])
    return ds @ k, ds.T @ q, p.T @ do


def _bwd_dv_untransposed(q, k, v, do, scale):
    dq, dk, dv = A.head_bwd(q, k, v, do, scale)
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    return dq, dk, (p @ np.eye(p.shape[1], do.shape[0])) @ do if p.shape[0] != p.shape[1] else p @ do


def _bwd_dk_uses_k(q, k, v, do, scale):
    dq, _, dv = A.head_bwd(q, k, v, do, scale)
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(1)[:, None])
    return dq, scale * ds.T @ (q + 0.5 * do), dv


def _bwd_d_over_columns(q, k, v, do, scale):
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(0)[None, :])
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_dq_swapped_kv(q, k, v, do, scale):
    q, k, v, do, p = _bwd_parts(q, k, v, do, scale)
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(1)[:, None])
    return scale * ds @ v, scale * ds.T @ q, p.T @ do


BWD_MUTANTS = [_bwd_drop_d, _bwd_wrong_sign, _bwd_no_scale, _bwd_dv_untransposed,
               _bwd_dk_uses_k, _bwd_d_over_columns, _bwd_dq_swapped_kv]


@pytest.mark.parametrize("mutant", BWD_MUTANTS, ids=lambda f: f.__name__)
def test_backward_pins_catch_planted_mistakes(mutant):
    errs = [pins.bwd_finite_differences(A.head_fwd, mutant, seeds=(0, 1)),
            pins.bwd_golden(mutant), pins.bwd_invariants(mutant)]
    assert max(errs) > 1e-5, errs


def _merge_no_renorm(o_parts, lse_parts):
    o, lse = A.lse_merge(o_parts, lse_parts)
    m = np.max(lse_parts, axis=0)
    w = np.exp(np.asarray(lse_parts) - np.where(np.isneginf(m), 0, m))
    return (w[..., None] * np.asarray(o_parts)).sum(0), lse


def _merge_lse_sum(o_parts, lse_parts):
    o, _ = A.lse_merge(o_parts, lse_parts)
    return o, np.asarray(lse_parts).sum(0)


def _merge_plain_mean(o_parts, lse_parts):
    _, lse = A.lse_merge(o_parts, lse_parts)
    return np.asarray(o_parts).mean(0), lse


def _merge_max_only(o_parts, lse_parts):
    o, _ = A.lse_merge(o_parts, lse_parts)
    return o, np.max(lse_parts, axis=0)


MERGE_MUTANTS = [_merge_no_renorm, _merge_lse_sum, _merge_plain_mean, _merge_max_only]


@pytest.mark.parametrize("mutant", MERGE_MUTANTS, ids=lambda f: f.__name__)
def test_merge_pins_catch_planted_mistakes(mutant):
    errs = [pins.merge_any_split(A.head_fwd, mutant), pins.merge_empty_parts(mutant)]
    assert max(errs) > 1e-6, errs


def _chunked_bwd_local_lse(q, k, v, do, scale, bounds, o, lse):
    # each chunk normalised on its own instead of by the merged LSE
    dq = np.zeros_like(np.asarray(q, dtype=float))
    dk = np.zeros_like(np.asarray(k, dtype=float))
    dv = np.zeros_like(np.asarray(v, dtype=float))
    for c in range(len(bounds) - 1):
        lo, hi = bounds[c], bounds[c + 1]
        if hi > lo:
            a, b, cc = A.head_bwd(q, k[lo:hi], v[lo:hi], do, scale)
            dq += a
            dk[lo:hi], dv[lo:hi] = b, cc
    return dq, dk, dv


def test_chunked_pin_catches_local_normalisation():
    assert pins.chunked_bwd_vs_unsplit(A.head_bwd, A.head_chunked_fwd,
                                       _chunked_bwd_local_lse) > 1e-6


def test_expr_helper_is_closed():
    assert math.isclose(pins._expr("ln(1+e)"), math.log(1 + math.e))

"""Helpers for the GPU parity tests: device upload and error metrics."""
import numpy as np
import torch

from exact_block_wise_amd.synth import bf16_bits

# Tolerances stated for the method's workloads: fp32 max relative error
# (infinity-norm, per tensor) 1e-5; bf16 outputs max abs 2e-2, LSE max abs
# 1e-3; gradients relative Frobenius error 1e-2.
TOL_F32_REL = 1e-5
TOL_O_ABS = 2e-2
TOL_LSE_ABS = 1e-3
TOL_GRAD_FRO = 1e-2


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload fp32 values (bf16-representable when dtype is bf16)."""
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(x, y) -> float:
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(y, np.float64))))


def rel_inf(x, y) -> float:
    y = np.asarray(y, np.float64)
    return max_abs(x, y) / max(float(np.max(np.abs(y))), 1e-300)


def rel_fro(x, y) -> float:
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    return float(np.linalg.norm((x - y).ravel()) / max(np.linalg.norm(y.ravel()), 1e-300))


def check_fwd(o, lse, o_ref, lse_ref, dtype, what=""):
    if dtype == "f32":
        eo, el = rel_inf(o, o_ref), rel_inf(lse, lse_ref)
        assert eo <= TOL_F32_REL and el <= TOL_F32_REL, f"{what} O rel {eo:.3g}, LSE rel {el:.3g}"
    else:
        eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
        assert eo <= TOL_O_ABS and el <= TOL_LSE_ABS, f"{what} O abs {eo:.3g}, LSE abs {el:.3g}"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    return eo, el


def check_grads(got, ref, dtype, what=""):
    """Relative error per gradient tensor.  A reference that is exactly zero
    (a closed-form zero, e.g. dQ = dK = 0 with a single key) has no relative
    error; there the GPU values must be at fp32 rounding level, |x| <= 1e-5."""
    errs = []
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(x)), f"{what} {name} not finite"
        if not np.any(np.asarray(y)):
            e = float(np.max(np.abs(x)))
            assert e <= 1e-5, f"{what} {name} should be 0, max |x| = {e:.3g}"
            errs.append(e)
            continue
        e = rel_inf(x, y) if dtype == "f32" else rel_fro(x, y)
        tol = TOL_F32_REL if dtype == "f32" else TOL_GRAD_FRO
        assert e <= tol, f"{what} {name} error {e:.3g} > {tol}"
        errs.append(e)
    return errs

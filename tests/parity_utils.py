"""Shared helpers for the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import numpy as np
import torch

# Parity bars against the float64 oracle: normwise max relative error per
# output tensor, max|x - ref| / max|ref|.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# Backward: every gradient is a float32 output computed in float32 from the
# same (exactly upcast) inputs as the oracle, so the bar is the float32 one
# whatever the input dtype.
TOL_BWD = 1e-4


def tol_for(dtype) -> float:
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def to_np(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach()
        if x.dtype == torch.bfloat16:
            x = x.float()
        return x.cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def rel_err(x, ref) -> float:
    x, ref = to_np(x), to_np(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def per_head_errors(x, ref, head_axes):
    """Normwise relative error of every (b, h) slice: max|x - ref| / max|ref|
    over the slice's other axes.  ``head_axes`` names the b and h axes
    (``(0, 2)`` for per-token ``[B, T, H, d]`` tensors, ``(0, 1)`` for state
    ``[B, H, dv, dk]``).  Returns an array ``[B, H]``."""
    x, ref = to_np(x), to_np(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    ab, ah = head_axes
    rest = tuple(a for a in range(x.ndim) if a not in head_axes)
    diff = np.abs(x - ref).max(axis=rest)
    den = np.abs(ref).max(axis=rest)
    err = diff / np.where(den > 0, den, 1.0)
    return err if ab < ah else err.T


def report_per_head(name, x, ref, head_axes, tol):
    """Print the worst (b, h) slices of a full-size comparison beside the
    normwise error, and assert every slice meets the bar as well."""
    e = per_head_errors(x, ref, head_axes)
    order = np.argsort(e, axis=None)[::-1][:3]
    worst = ", ".join("(b=%d,h=%d) %.3e" % (*np.unravel_index(i, e.shape), e.flat[i]) for i in order)
    print("  %-22s per-(b,h) max %.3e over %d heads; worst %s" % (name, e.max(), e.size, worst), flush=True)
    assert e.max() <= tol, "%s: worst (b,h) rel err %.3e > %.1e" % (name, e.max(), tol)


def assert_close(name, x, ref, tol, log=None):
    e = rel_err(x, ref)
    if log is not None:
        log[name] = e
    print("  %-22s max normwise rel err %.3e (bar %.0e)" % (name, e, tol), flush=True)
    assert np.isfinite(to_np(x)).all(), "%s has non-finite values" % name
    assert e <= tol, "%s: rel err %.3e > %.1e" % (name, e, tol)


def to_device(inp: dict, dev) -> dict:
    return {n: (x.to(dev) if isinstance(x, torch.Tensor) else x) for n, x in inp.items()}


def gpu_args(inp: dict):
    return (inp["q"], inp["k"], inp["v"], inp["beta"], inp["dt"], inp["A"], inp["I_prior"])

"""Shared parity helpers for the GPU tests (comparison only, no attention math).

Tolerances: |gpu - oracle| <= atol + rtol * |oracle| for every element.
  fp32 inputs:       atol 1e-3, rtol 1e-2 -- the stricter published pair (page
                     "Shape-Aware Attention", section "What it does");
  bf16/fp16 inputs:  atol 2e-2, rtol 2e-2 -- the pages give no half-precision
                     pair for a single attention call; this pair is derived in
                     the design notes from the bf16 rounding of the
                     probabilities fed to the P.V product (unit roundoff 2^-8,
                     so the error is at most ~2^-8 * max|v| ~ 1.6e-2 for
                     |v| <= 4, usually far less) plus the output rounding.
Any NaN or Inf fails.
"""
import numpy as np

TOL = {"f32": (1e-3, 1e-2), "f16": (2e-2, 2e-2), "bf16": (2e-2, 2e-2)}


def compare(got, ref, dtype, what=""):
    """Assert elementwise closeness; returns (max_abs_err, worst_ratio)."""
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[worst] <= 1.0, (f"{what}: element {worst} got {got[worst]} ref {ref[worst]} "
                                 f"err {err[worst]:.3e} > bound {bound[worst]:.3e}")
    return float(err.max()), float(ratio.max())

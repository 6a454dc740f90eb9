"""Acceptance check shared by the parity tests.

Every output element must satisfy |D - ref| <= tau * bound with
bound = sum_k |a*b| + |c|; tau = 1e-4 for fp32 outputs and 8e-3 for bf16
outputs.  NaN or Inf anywhere fails.
"""
import numpy as np

TAU = {"f32": 1e-4, "bf16": 8e-3}


def check_close(d, ref, bound, d_dtype, what=""):
    d = np.asarray(d, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    assert d.shape == ref.shape, (what, d.shape, ref.shape)
    assert np.all(np.isfinite(d)), f"{what}: non-finite outputs"
    err = np.abs(d - ref)
    lim = TAU[d_dtype] * bound
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[:5]
        worst = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
            f"first {idx.tolist()}; worst {worst}: d={d[worst]} ref={ref[worst]} "
            f"bound={bound[worst]}")
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0

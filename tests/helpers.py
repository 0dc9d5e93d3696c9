"""Shared helpers for the GPU parity tests (tolerances, cache set-up)."""
import numpy as np

# Tolerance of the decode attention against the f64 oracle, per (sequence,
# head) output row: max_d |gpu - ref| <= TOL * max_d |ref|.  1e-4 for f32 K/V,
# 2e-2 for bf16 K/V.  Rows the oracle sets to zero must be exactly zero.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def row_rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(gpu - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return num / den


def assert_attention_close(gpu, ref, dtype, what=""):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    zero_rows = np.all(ref == 0.0, axis=-1)
    if zero_rows.any():
        assert np.all(gpu[zero_rows] == 0.0), f"{what}: rows the oracle zeroes are not zero"
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = row_rel_err(gpu, ref)
    worst = float(err.max(initial=0.0))
    assert worst <= TOL[dtype], f"{what}: worst row-relative error {worst:.3e} > {TOL[dtype]}"
    return worst

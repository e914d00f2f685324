"""Parity metrics applied between a GPU result and the float64 oracle.  TEST INFRASTRUCTURE ONLY.

Tolerances (stated for the differential-attention forward pass):
  * fp32 inputs: row-normwise relative error  max_rows ||x - r||_inf / ||r||_inf  <= 1e-5
    (element-wise relative error is ill-posed near zero, so the row's own scale is used).
  * bf16 inputs with fp32 accumulation, compared after normalisation: max |x - r| <= 2e-2 and
    at least 99.9 % of elements with |x - r| <= 1e-2.  The V1 output is already RMS-normalised
    (times 1 - lambda_init) and is compared as is.  V2 and decode outputs carry no norm, so
    both sides are divided by the RMS of the oracle row first; raw V2 outputs are ~0.01-0.02 in
    size at the benchmark shapes and an absolute 2e-2 bound on them would be vacuous.
"""

from __future__ import annotations

import numpy as np

FP32_ROW_REL_TOL = 1e-5
BF16_MAX_ABS_TOL = 2e-2
BF16_ELEM_TOL = 1e-2
BF16_MIN_FRAC_WITHIN = 0.999


def row_rel_error(x, ref) -> float:
    """max over rows of ||x - ref||_inf / ||ref||_inf (rows = last axis)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if x.size == 0:
        return 0.0
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den))


def normalise_by_ref_rms(x, ref):
    """Divide both arrays row by row by the RMS of the reference row."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    rms = np.where(rms > 0, rms, 1.0)
    return x / rms, ref / rms


def bf16_stats(x, ref, normalise: bool = False) -> dict:
    """max abs error and fraction of elements within BF16_ELEM_TOL (optionally RMS-normalised)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if normalise:
        x, ref = normalise_by_ref_rms(x, ref)
    if x.size == 0:
        return {"max_abs": 0.0, "frac_within": 1.0, "n": 0, "finite": True}
    err = np.abs(x - ref)
    finite = bool(np.all(np.isfinite(x)))
    return {
        "max_abs": float(np.max(err)) if finite else float("inf"),
        "frac_within": float(np.mean(err <= BF16_ELEM_TOL)),
        "n": int(x.size),
        "finite": finite,
    }


def bf16_ok(stats: dict) -> bool:
    return (stats["finite"] and stats["max_abs"] <= BF16_MAX_ABS_TOL
            and stats["frac_within"] >= BF16_MIN_FRAC_WITHIN)

"""Pins of the parity metrics in ``oracle/compare.py`` on hand-computed arrays (CPU).

Every GPU parity decision goes through ``row_rel_error``, ``normalise_by_ref_rms``, ``bf16_stats``
and ``bf16_ok``, so a slip there would loosen every GPU test at once.  The checks below fix each
function on arrays whose answer is worked out by hand:

* the row-normwise relative error divides each row's max error by that *reference* row's max;
* the normalisation divides both rows by the RMS of the *reference* (oracle) row, before the
  error is taken, and leaves an all-zero reference row unscaled;
* an element with error exactly 1e-2 counts as within; 999 of 1000 within is exactly the
  99.9 % bar and passes, 998 of 1000 fails; a max error of exactly 2e-2 passes, just above fails;
* a non-finite GPU value fails however close the rest is.

``test_planted_slips_are_caught`` runs the same checks on copies of the module with one plausible
slip each (normalising by the GPU row, normalising after taking the error, ``<`` for ``<=`` at
either boundary, the mean instead of the max over rows, ignoring non-finite values) and requires
every copy to fail at least one check.
"""

from __future__ import annotations

import types

import numpy as np
import pytest

from oracle import compare


# ------------------------------------------------------------------------------------------------
# the checks, written against a module-like object so that planted slips can be run through them
# ------------------------------------------------------------------------------------------------

def check_row_rel_error(m):
    ref = np.array([[1.0, -4.0, 2.0], [0.5, 0.25, -0.5]])
    x = ref + np.array([[0.0, 0.02, -0.01], [0.001, 0.0, 0.0]])
    # row 0: 0.02 / 4 = 5e-3; row 1: 1e-3 / 0.5 = 2e-3 -> max over rows 5e-3
    assert m.row_rel_error(x, ref) == pytest.approx(5e-3, rel=1e-12)
    # the row with the smaller reference norm must be the one that decides here
    x2 = ref + np.array([[0.0, 0.004, 0.0], [0.0, 0.0, 0.004]])
    # row 0: 0.004 / 4 = 1e-3; row 1: 0.004 / 0.5 = 8e-3
    assert m.row_rel_error(x2, ref) == pytest.approx(8e-3, rel=1e-12)
    # an all-zero reference row is measured in absolute terms
    z = np.zeros((1, 4))
    assert m.row_rel_error(z + 3e-6, z) == pytest.approx(3e-6, rel=1e-12)
    assert m.row_rel_error(ref, ref) == 0.0
    with pytest.raises(ValueError):
        m.row_rel_error(np.zeros((2, 3)), np.zeros((3, 2)))


def check_normalise(m):
    ref = np.array([[3.0, 4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 0.0]])
    x = np.array([[6.0, 8.0, 0.0, 0.0], [2.0, 0.0, 1.0, 1.0], [0.5, 0.0, 0.0, 0.0]])
    xn, rn = m.normalise_by_ref_rms(x, ref)
    # RMS of row 0 of ref = sqrt((9 + 16) / 4) = 2.5; of row 1 = 1; row 2 has RMS 0 -> unscaled
    np.testing.assert_allclose(rn[0], [1.2, 1.6, 0.0, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(xn[0], [2.4, 3.2, 0.0, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(xn[1], x[1], rtol=0, atol=0)
    np.testing.assert_allclose(xn[2], x[2], rtol=0, atol=0)
    assert np.all(np.isfinite(rn)) and np.all(np.isfinite(xn))


def check_bf16_stats(m):
    # un-normalised: one element exactly at the 1e-2 element bound counts as within
    ref = np.zeros((1, 4))
    x = np.array([[0.01, 0.0, -0.005, 0.0]])
    st = m.bf16_stats(x, ref)
    assert st["n"] == 4 and st["finite"]
    assert st["max_abs"] == pytest.approx(0.01, rel=1e-15)
    assert st["frac_within"] == 1.0
    # normalised: errors are measured after dividing by the reference row's RMS (here 2)
    ref = np.array([[2.0, -2.0, 2.0, -2.0]])
    x = ref + np.array([[0.03, 0.0, 0.0, 0.0]])   # raw error 0.03 -> 0.015 after normalising
    st = m.bf16_stats(x, ref, normalise=True)
    assert st["max_abs"] == pytest.approx(0.015, rel=1e-12)
    assert st["frac_within"] == pytest.approx(0.75)
    st_raw = m.bf16_stats(x, ref)
    assert st_raw["max_abs"] == pytest.approx(0.03, rel=1e-12)
    # empty input
    st = m.bf16_stats(np.zeros((0, 3)), np.zeros((0, 3)))
    assert st["n"] == 0 and m.bf16_ok(st)


def check_bf16_ok_boundaries(m):
    ref = np.zeros((10, 100))
    # 999 of 1000 within 1e-2, the other at exactly the 2e-2 max bound: passes
    x = ref.copy()
    x[3, 7] = 0.02
    st = m.bf16_stats(x, ref)
    assert st["frac_within"] == pytest.approx(0.999, abs=0)
    assert m.bf16_ok(st), st
    # two elements out: 99.8 % -> fails
    x[5, 5] = 0.015
    assert not m.bf16_ok(m.bf16_stats(x, ref))
    # one element just above the max bound: fails even though 99.9 % are within
    x = ref.copy()
    x[0, 0] = 0.0200001
    assert not m.bf16_ok(m.bf16_stats(x, ref))
    # every element at exactly the element bound: all within
    x = ref + 0.01
    st = m.bf16_stats(x, ref)
    assert st["frac_within"] == 1.0 and m.bf16_ok(st)


def check_non_finite(m):
    ref = np.ones((4, 8))
    for bad in (np.nan, np.inf, -np.inf):
        x = ref.copy()
        x[2, 3] = bad
        st = m.bf16_stats(x, ref, normalise=True)
        assert not st["finite"]
        assert not m.bf16_ok(st)
        assert not m.bf16_ok(m.bf16_stats(x, ref))


CHECKS = (check_row_rel_error, check_normalise, check_bf16_stats, check_bf16_ok_boundaries,
          check_non_finite)


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_compare_module(check):
    check(compare)


def test_tolerances_are_the_stated_ones():
    assert compare.FP32_ROW_REL_TOL == 1e-5
    assert compare.BF16_MAX_ABS_TOL == 2e-2
    assert compare.BF16_ELEM_TOL == 1e-2
    assert compare.BF16_MIN_FRAC_WITHIN == 0.999


# ------------------------------------------------------------------------------------------------
# planted slips
# ------------------------------------------------------------------------------------------------

def _variant(**over):
    ns = {k: getattr(compare, k) for k in ("FP32_ROW_REL_TOL", "BF16_MAX_ABS_TOL", "BF16_ELEM_TOL",
                                           "BF16_MIN_FRAC_WITHIN", "row_rel_error",
                                           "normalise_by_ref_rms", "bf16_stats", "bf16_ok")}
    ns.update(over)
    return types.SimpleNamespace(**ns)


def _stats_factory(normaliser=None, within=lambda e, t: e <= t, after=False, check_finite=True):
    """A bf16_stats written like the real one, with one part swapped for a slip."""
    def stats(x, ref, normalise=False):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if x.shape != ref.shape:
            raise ValueError("shape mismatch")
        if x.size == 0:
            return {"max_abs": 0.0, "frac_within": 1.0, "n": 0, "finite": True}
        if normalise and not after:
            x, ref = (normaliser or compare.normalise_by_ref_rms)(x, ref)
        err = np.abs(x - ref)
        if normalise and after:
            # slip: the error is scaled by the RMS of the GPU row after it is taken
            rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
            err = err / np.where(rms > 0, rms, 1.0)
        finite = bool(np.all(np.isfinite(x))) if check_finite else True
        return {"max_abs": float(np.nanmax(err)) if finite else float("inf"),
                "frac_within": float(np.mean(within(err, compare.BF16_ELEM_TOL))),
                "n": int(x.size), "finite": finite}
    return stats


def _norm_by_gpu(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    rms = np.where(rms > 0, rms, 1.0)
    return x / rms, ref / rms


def _norm_by_max(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mx = np.max(np.abs(ref), axis=-1, keepdims=True)
    mx = np.where(mx > 0, mx, 1.0)
    return x / mx, ref / mx


def _row_rel_mean(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.mean(num / np.where(den > 0, den, 1.0)))


def _row_rel_global(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


def _ok_strict_frac(st):
    return st["finite"] and st["max_abs"] <= 2e-2 and st["frac_within"] > 0.999


def _ok_strict_max(st):
    return st["finite"] and st["max_abs"] < 2e-2 and st["frac_within"] >= 0.999


def _ok_ignores_finite(st):
    return st["max_abs"] <= 2e-2 and st["frac_within"] >= 0.999


SLIPS = {
    "normalise by the GPU row": dict(normalise_by_ref_rms=_norm_by_gpu,
                                     bf16_stats=_stats_factory(normaliser=_norm_by_gpu)),
    "normalise by the row max": dict(normalise_by_ref_rms=_norm_by_max,
                                     bf16_stats=_stats_factory(normaliser=_norm_by_max)),
    "normalise after the error": dict(bf16_stats=_stats_factory(after=True)),
    "< at the element bound": dict(bf16_stats=_stats_factory(within=lambda e, t: e < t)),
    "> at the 99.9 % bar": dict(bf16_ok=_ok_strict_frac),
    "< at the max bound": dict(bf16_ok=_ok_strict_max),
    "non-finite ignored": dict(bf16_stats=_stats_factory(check_finite=False), bf16_ok=_ok_ignores_finite),
    "mean over rows": dict(row_rel_error=_row_rel_mean),
    "one global scale": dict(row_rel_error=_row_rel_global),
}


@pytest.mark.parametrize("slip", sorted(SLIPS))
def test_planted_slips_are_caught(slip):
    m = _variant(**SLIPS[slip])
    failed = 0
    for check in CHECKS:
        try:
            check(m)
        except (AssertionError, ValueError, FloatingPointError):
            failed += 1
    assert failed > 0, f"slip {slip!r} passed every check of the parity metrics"

"""GPU parity at the method's lambda extremes.

ai-engineering.academy "Atención Diferencial (V2)", section "La idea diferencial": lambda is a
learnable scalar that may be negative; section "Ejercicios" (exercise 4) takes lambda = 0 (plain
softmax attention of the first map) and lambda = 1 (full subtraction).  The lambda vectors of the
workloads keep lambda within about +-0.1 of lambda_init, so these cases pass lambda directly
through the ``lambda_override`` hook of the C ABI: lambda in {-0.5, 0, 1, 1.5} for V1 (normalised
and core), V1 fp32, V2 and both decode steps, and identical branches with lambda = 1, whose
output is exactly zero in exact arithmetic (each row of A1 - A2 is the zero row).

Identical branches make the two branch computations bit-identical on the GPU as well; what can
remain of the difference is the rounding residual of one product when the compiler fuses the
subtraction into a fused multiply-add (about 2^-24 of the branch output), which the V1 norm maps
to at most that residual over sqrt(eps).  The test bounds the output by 1e-4, far below the O(1)
of any slip (a wrong branch, sign or lambda).  The core without the norm (flag DA_V1_NO_NORM) has no fixed scale and is checked
componentwise against the error bf16 weights allow: |err| <= 2^-8 (|A1||V| + |lambda||A2||V| + |ref|).
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import dev, f64, log

pytestmark = pytest.mark.gpu

LAMBDAS = (-0.5, 0.0, 1.0, 1.5)


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _lam(value, n):
    import torch

    return torch.full((n,), float(value), dtype=torch.float32, device="cuda")


def _v1(da, t, lam, layer, dtype="bf16", flags=0, causal=True):
    import torch

    o = da.diffattn_fwd_v1(*(dev(t[k], dtype) for k in ("q1", "q2", "k1", "k2", "v")), layer=layer,
                           lambda_override=_lam(lam, t["q1"].shape[1]), flags=flags, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _core_bound(t, lam, ref, causal=True):
    """2^-8 (|A1||V| + |lambda||A2||V| + |ref|) per element, per (b, h)."""
    q1, q2, k1, k2, v = (f64(t[k]) for k in ("q1", "q2", "k1", "k2", "v"))
    out = np.empty_like(ref)
    for b in range(q1.shape[0]):
        for h in range(q1.shape[1]):
            a1, a2, _ = oracle.diff_maps(q1[b, h], k1[b, h], q2[b, h], k2[b, h], lam, causal)
            mag = np.abs(a1) @ np.abs(v[b, h]) + abs(lam) * (np.abs(a2) @ np.abs(v[b, h]))
            out[b, h] = 2.0 ** -8 * (mag + np.abs(ref[b, h]))
    return out


@pytest.mark.parametrize("lam", LAMBDAS)
def test_v1_bf16_lambda_extremes(da, lam):
    layer = 5
    t = wl.make_v1(2, 2, 333, 64, "bf16", seed=1400, layers=(layer,))
    got = _v1(da, t, lam, layer)
    ref = oracle.diff_attn_v1(*(f64(t[k]) for k in ("q1", "q2", "k1", "k2", "v")), np.full(2, lam),
                              oracle.lambda_init(layer), True, 1e-5)
    st = compare.bf16_stats(got, ref)
    log(f"v1 bf16 lambda={lam}: {st}")
    assert compare.bf16_ok(st), st
    core = _v1(da, t, lam, layer, flags=da.DA_V1_NO_NORM)
    cref = oracle.diff_attn_v1(*(f64(t[k]) for k in ("q1", "q2", "k1", "k2", "v")), np.full(2, lam),
                               oracle.lambda_init(layer), True, 1e-5, norm=False)
    worst = float(np.max(np.abs(core - cref) / _core_bound(t, lam, cref)))
    log(f"  core worst err / bound {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("lam", LAMBDAS)
def test_v1_fp32_lambda_extremes(da, lam):
    layer = 2
    t = wl.make_v1(1, 2, 150, 64, "f32", seed=1401, layers=(layer,))
    got = _v1(da, t, lam, layer, dtype="f32", causal=False)
    ref = oracle.diff_attn_v1(*(t[k].astype(np.float64) for k in ("q1", "q2", "k1", "k2", "v")),
                              np.full(2, lam), oracle.lambda_init(layer), False, 1e-5)
    err = compare.row_rel_error(got, ref)
    log(f"v1 fp32 lambda={lam}: row-relative error {err:.3e}")
    assert err <= compare.FP32_ROW_REL_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, 1])
def test_v1_identical_branches_full_subtraction_is_zero(da, dtype, flags):
    """Q2 = Q1, K2 = K1, lambda = 1: A1 - A2 = 0, so the exact output is zero."""
    layer = 7
    t = wl.make_v1(2, 3, 290, 64, dtype, seed=1402, layers=(layer,))
    t["q2"], t["k2"] = t["q1"].copy(), t["k1"].copy()
    got = _v1(da, t, 1.0, layer, dtype=dtype, flags=flags)
    ref = oracle.diff_attn_v1(*(f64(t[k], dtype) for k in ("q1", "q2", "k1", "k2", "v")),
                              np.ones(3), oracle.lambda_init(layer), True, 1e-5, norm=not flags)
    assert np.max(np.abs(ref)) == 0.0
    log(f"v1 {dtype} identical branches flags={flags}: max |out| {np.max(np.abs(got)):.3e}")
    assert np.max(np.abs(got)) <= 1e-4


@pytest.mark.parametrize("lam", LAMBDAS)
def test_v2_lambda_extremes(da, lam):
    import torch

    t = wl.make_v2(1, 4, 2, 300, 128, "bf16", seed=1403, layers=(24,))
    q = dev(t["q"])
    o = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], dev(t["k"]), dev(t["v"]), layer=24,
                           lambda_override=_lam(lam, 4))
    torch.cuda.synchronize()
    ref = oracle.diff_attn_v2(f64(t["q"]), f64(t["k"]), f64(t["v"]), np.full(4, lam), True)
    st = compare.bf16_stats(o.float().cpu().numpy(), ref, normalise=True)
    log(f"v2 lambda={lam}: {st}")
    assert compare.bf16_ok(st), st


def test_v2_identical_heads_full_subtraction_is_zero(da):
    import torch

    t = wl.make_v2(2, 4, 2, 257, 128, "bf16", seed=1404, layers=(24,))
    t["q"][:, 1::2] = t["q"][:, 0::2]
    q = dev(t["q"])
    for window in (0, 50):
        o = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], dev(t["k"]), dev(t["v"]), layer=24,
                               lambda_override=_lam(1.0, 4), window=window)
        torch.cuda.synchronize()
        worst = float(o.float().abs().max())
        log(f"v2 identical heads window={window}: max |out| {worst:.3e}")
        assert worst <= 1e-4, window


@pytest.mark.parametrize("lam", LAMBDAS)
def test_decode_lambda_extremes(da, lam):
    import torch

    t = wl.make_decode(2, 4, 2, 1500, 128, "bf16", seed=1405, layers=(24,))
    q = dev(t["q"])
    o = da.diffattn_decode(q[:, 0::2], q[:, 1::2], dev(t["kcache"]), dev(t["vcache"]), layer=24,
                           lambda_override=_lam(lam, 4))
    torch.cuda.synchronize()
    ref = oracle.diff_decode_v2(f64(t["q"]), f64(t["kcache"]), f64(t["vcache"]), np.full(4, lam))
    st = compare.bf16_stats(o.float().cpu().numpy(), ref, normalise=True)
    log(f"decode lambda={lam}: {st}")
    assert compare.bf16_ok(st), st


@pytest.mark.parametrize("lam", LAMBDAS)
def test_decode_v1_lambda_extremes(da, lam):
    import torch

    layer = 12
    t = wl.make_decode_v1(2, 3, 1300, 64, "bf16", seed=1406, layers=(layer,))
    o = da.diffattn_decode_v1(*(dev(t[k]) for k in ("q1", "q2", "k1cache", "k2cache", "vcache")),
                              layer=layer, lambda_override=_lam(lam, 3))
    torch.cuda.synchronize()
    ref = oracle.diff_decode_v1(*(f64(t[k]) for k in ("q1", "q2", "k1cache", "k2cache", "vcache")),
                                np.full(3, lam), oracle.lambda_init(layer))
    st = compare.bf16_stats(o.float().cpu().numpy(), ref)
    log(f"decode v1 lambda={lam}: {st}")
    assert compare.bf16_ok(st), st


def test_decode_v1_identical_branches_is_zero(da):
    import torch

    t = wl.make_decode_v1(2, 2, 900, 64, "bf16", seed=1407, layers=(3,))
    t["q2"], t["k2cache"] = t["q1"].copy(), t["k1cache"].copy()
    o = da.diffattn_decode_v1(*(dev(t[k]) for k in ("q1", "q2", "k1cache", "k2cache", "vcache")),
                              layer=3, lambda_override=_lam(1.0, 2))
    torch.cuda.synchronize()
    worst = float(o.float().abs().max())
    log(f"decode v1 identical branches: max |out| {worst:.3e}")
    assert worst <= 1e-4

"""GPU parity of the causal sliding-window prefill (row i sees keys i - W + 1 .. i) against the
float64 CPU oracle, for the V1 (bf16 and fp32) and V2 layouts."""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import dev, dev_lambda, f64, log, oracle_lambda, parallel_map

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _run_v1(da, t, dtype, layer, window, flags=0):
    import torch

    lv = dev_lambda(t["lambda"][layer])
    args = [dev(t[k], dtype) for k in ("q1", "q2", "k1", "k2", "v")]
    o = da.diffattn_fwd_v1(*args, *lv, layer=layer, window=window, flags=flags)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _oracle_v1(t, dtype, layer, window, norm=True, rows=None, heads=None, batches=None):
    lam = oracle_lambda(t["lambda"][layer], layer)
    return oracle.diff_attn_v1(*(f64(t[k], dtype) for k in ("q1", "q2", "k1", "k2", "v")), lam,
                               oracle.lambda_init(layer), True, 1e-5, norm, rows=rows,
                               heads=heads, batches=batches, window=window)


@pytest.mark.parametrize("B,H,N,window", [
    (1, 2, 100, 1),       # each row sees only itself
    (1, 2, 100, 31),
    (2, 1, 200, 32),      # window = one tile
    (1, 3, 257, 33),
    (1, 2, 300, 64),      # window = one row block
    (1, 2, 129, 1000),    # window longer than the sequence: plain causal
    (1, 1, 513, 100),
])
def test_window_v1_bf16_full_compare(da, B, H, N, window):
    log(f"v1 window B={B} H={H} N={N} W={window}")
    t = wl.make_v1(B, H, N, 64, "bf16", seed=N + window, layers=(12,))
    got = _run_v1(da, t, "bf16", 12, window)
    st = compare.bf16_stats(got, _oracle_v1(t, "bf16", 12, window))
    log(f"  stats {st}")
    assert compare.bf16_ok(st), st


@pytest.mark.parametrize("N,window", [(128, 1), (128, 17), (200, 64)])
def test_window_v1_fp32(da, N, window):
    log(f"v1 fp32 window N={N} W={window}")
    t = wl.make_v1(1, 2, N, 64, "f32", seed=7 + window, layers=(3,))
    got = _run_v1(da, t, "f32", 3, window)
    err = compare.row_rel_error(got, _oracle_v1(t, "f32", 3, window))
    log(f"  row-rel {err:.3e}")
    assert err <= compare.FP32_ROW_REL_TOL


def test_window_of_one_core_is_one_minus_lambda_times_v(da):
    """W = 1 with the norm off: both maps are the identity, the core is (1 - lambda) V."""
    log("v1 window 1 core")
    t = wl.make_v1(1, 4, 150, 64, "bf16", seed=12, layers=(5,))
    got = _run_v1(da, t, "bf16", 5, 1, flags=da.DA_V1_NO_NORM)
    lam = oracle_lambda(t["lambda"][5], 5)
    ref = (1 - lam)[None, :, None, None] * f64(t["v"])
    st = compare.bf16_stats(got, ref, normalise=True)
    assert compare.bf16_ok(st), st


def test_window_longer_than_sequence_equals_causal(da):
    import torch

    t = wl.make_v1(1, 2, 300, 64, "bf16", seed=4, layers=(12,))
    a = _run_v1(da, t, "bf16", 12, 300)
    lv = dev_lambda(t["lambda"][12])
    args = [dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    b = da.diffattn_fwd_v1(*args, *lv, layer=12).float().cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("B,P,Hkv,N,window", [
    (1, 4, 2, 200, 50),
    (1, 16, 8, 333, 64),
    (2, 2, 1, 130, 1),
    (1, 2, 2, 257, 95),
])
def test_window_v2_full_compare(da, B, P, Hkv, N, window):
    import torch

    log(f"v2 window B={B} P={P} Hkv={Hkv} N={N} W={window}")
    t = wl.make_v2(B, P, Hkv, N, 128, "bf16", seed=N + window + P, layers=(24,))
    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][24])
    got = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], dev(t["k"]), dev(t["v"]), *lv, layer=24,
                             window=window).float().cpu().numpy()
    torch.cuda.synchronize()
    lam = oracle_lambda(t["lambda"][24], 24)
    ref = oracle.diff_attn_v2(f64(t["q"]), f64(t["k"]), f64(t["v"]), lam, True, window=window)
    st = compare.bf16_stats(got, ref, normalise=True)
    log(f"  stats {st}")
    assert compare.bf16_ok(st), st


def test_window_workload_4k_every_row(da):
    """The sliding-window workload (B=4, H=16, N=4096, W=1024), one launch: every row of every
    (batch, head) slice against the oracle, element by element."""
    cfg, t = wl.make("v1_swa_4k")
    layer, window = cfg["layers"][0], cfg["window"]
    B, H = cfg["B"], cfg["H"]
    log("v1 window W=1024 N=4096 (full launch, every row)")
    got = _run_v1(da, t, "bf16", layer, window)
    assert np.isfinite(got).all()
    lam = oracle_lambda(t["lambda"][layer], layer)

    def one(bh):
        b, h = divmod(bh, H)
        sl = [f64(t[k][b:b + 1, h:h + 1]) for k in ("q1", "q2", "k1", "k2", "v")]
        ref = oracle.diff_attn_v1(*sl, lam[h:h + 1], oracle.lambda_init(layer), True, 1e-5,
                                  window=window)[0, 0]
        return b, h, compare.bf16_stats(got[b, h], ref)

    worst = None
    for b, h, st in parallel_map(one, range(B * H)):
        assert compare.bf16_ok(st), (b, h, st)
        worst = st if worst is None or st["max_abs"] > worst["max_abs"] else worst
    log(f"  64 slices ok, worst {worst}")

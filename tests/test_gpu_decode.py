"""GPU parity of the V2 decode step against the float64 CPU oracle (compared after dividing both
sides by the RMS of the oracle row, as V2 carries no normalisation)."""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import beyond_output_rounding, dev, dev_lambda, f64, log, merge_stats, oracle_lambda, parallel_map

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _run_decode(da, t, layer, num_splits=0, kc=None, vc=None):
    import torch

    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][layer])
    kc = dev(t["kcache"]) if kc is None else kc
    vc = dev(t["vcache"]) if vc is None else vc
    o = da.diffattn_decode(q[:, 0::2], q[:, 1::2], kc, vc, *lv, layer=layer, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


@pytest.mark.parametrize("B,P,Hkv,L,splits", [
    (1, 1, 1, 1, 0),        # G = 2, a single cache row
    (2, 2, 1, 100, 0),      # G = 4, one partial block
    (1, 4, 1, 256, 0),      # G = 8, exactly one block
    (1, 8, 1, 1000, 3),     # G = 16, ragged blocks across 3 splits
    (3, 16, 8, 5000, 0),    # the workload's head layout
    (2, 16, 8, 5000, 1),    # same, unsplit
    (1, 4, 2, 2049, 7),
    (2, 4, 1, 3000, 2),     # G = 8 over several blocks per split
])
def test_decode_full_compare(da, B, P, Hkv, L, splits):
    log(f"decode B={B} P={P} Hkv={Hkv} L={L} splits={splits}")
    t = wl.make_decode(B, P, Hkv, L, 128, "bf16", seed=L + P, layers=(24,))
    got = _run_decode(da, t, 24, splits)
    lam = oracle_lambda(t["lambda"][24], 24)
    ref = oracle.diff_decode_v2(f64(t["q"]), f64(t["kcache"]), f64(t["vcache"]), lam)
    st = compare.bf16_stats(got, ref, normalise=True)
    log(f"  stats {st}")
    assert compare.bf16_ok(st), st


def test_decode_split_count_invariance(da):
    log("decode split invariance L=3000")
    t = wl.make_decode(2, 16, 8, 3000, 128, "bf16", seed=5, layers=(24,))
    outs = [_run_decode(da, t, 24, s) for s in (1, 2, 5, 12)]
    rms = np.sqrt(np.mean(outs[0] ** 2, axis=-1, keepdims=True))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0]) / rms) < 2e-2


def test_decode_matches_prefill_last_row(da):
    """The decode step equals the last row of the V2 prefill over the same tokens."""
    import torch

    log("decode vs prefill last row N=400")
    t = wl.make_v2(2, 4, 2, 400, 128, "bf16", seed=21, layers=(24,))
    q = dev(t["q"])
    k, v = dev(t["k"]), dev(t["v"])
    lv = dev_lambda(t["lambda"][24])
    pre = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], k, v, *lv, layer=24)
    ql = q[:, :, -1, :].contiguous()
    dec = da.diffattn_decode(ql[:, 0::2], ql[:, 1::2], k, v, *lv, layer=24)
    torch.cuda.synchronize()
    a = pre[:, :, -1].float().cpu().numpy()
    b = dec.float().cpu().numpy()
    # two bf16 results, each within 2e-2 (relative to the row RMS) of the exact value
    rms = np.sqrt(np.mean(a * a, axis=-1, keepdims=True))
    assert np.max(np.abs(a - b) / rms) < 4e-2


@pytest.mark.timeout(900)
def test_decode_workload_32k_every_sequence(da):
    """Full decode workload (B=64, 32 query heads / 8 KV heads, D=128, L=32768), one launch,
    every sequence against the oracle (one sequence per oracle call)."""
    cfg, t = wl.make("v2_decode_32k")
    layer = cfg["layers"][0]
    log("decode B=64 P=16 Hkv=8 L=32768 (full launch, every sequence)")
    got = _run_decode(da, t, layer)
    assert np.isfinite(got).all()
    lam = oracle_lambda(t["lambda"][layer], layer)

    def one(b):
        ref = oracle.diff_decode_v2(f64(t["q"][b:b + 1]), f64(t["kcache"][b:b + 1]),
                                    f64(t["vcache"][b:b + 1]), lam)
        return b, compare.bf16_stats(got[b:b + 1], ref, normalise=True), beyond_output_rounding(got[b:b + 1], ref)

    res = parallel_map(one, range(cfg["B"]))
    st = merge_stats([r[1] for r in res])
    excess = max(r[2] for r in res)
    log(f"  {cfg['B']} sequences: {st}; largest error beyond the bf16 output rounding "
        f"{excess:.2e} of the row RMS")
    assert compare.bf16_ok(st), st
    # every step before the final bf16 store runs in fp32: past the store's own rounding, what is
    # left is fp32 summation over the cache
    assert excess <= 2e-3

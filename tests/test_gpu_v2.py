"""GPU parity of the V2 prefill (paired query heads over shared GQA KV heads) against the float64
CPU oracle.  V2 has no normalisation, so both sides are divided by the RMS of the oracle row
before the bf16 tolerance (max |err| <= 2e-2, >= 99.9 % within 1e-2) is applied."""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import dev, dev_lambda, f64, log, oracle_lambda, parallel_map, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _run_v2(da, t, layer, causal=True, lambda_out=None):
    import torch

    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][layer])
    o = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], dev(t["k"]), dev(t["v"]), *lv, layer=layer,
                           causal=causal, lambda_out=lambda_out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _oracle_v2(t, layer, causal=True, rows=None, pairs=None, batches=None):
    lam = oracle_lambda(t["lambda"][layer], layer)
    return oracle.diff_attn_v2(f64(t["q"]), f64(t["k"]), f64(t["v"]), lam, causal, rows=rows,
                               pairs=pairs, batches=batches)


@pytest.mark.parametrize("B,P,Hkv,N,causal", [
    (1, 1, 1, 1, True),       # one pair per KV head, one key
    (1, 3, 3, 100, True),
    (2, 2, 1, 64, False),     # two pairs per KV head
    (1, 4, 2, 129, True),     # ragged tail one past a 64-row block
    (2, 8, 2, 200, True),     # four pairs per KV head
    (1, 16, 8, 333, True),    # the workload's head layout at a short length
    (1, 6, 2, 150, False),    # three pairs per KV head
    (1, 16, 1, 97, True),     # sixteen pairs over a single KV head
])
def test_v2_full_compare(da, B, P, Hkv, N, causal):
    log(f"v2 B={B} P={P} Hkv={Hkv} N={N} causal={causal}")
    t = wl.make_v2(B, P, Hkv, N, 128, "bf16", seed=N + 13 * P + Hkv, layers=(24,))
    got = _run_v2(da, t, 24, causal)
    ref = _oracle_v2(t, 24, causal)
    st = compare.bf16_stats(got, ref, normalise=True)
    log(f"  stats {st}")
    assert compare.bf16_ok(st), st


def test_v2_values_beyond_fp16_range(da):
    """P.V runs in fp16 except for V tiles holding a value fp16 cannot represent; those tiles
    take the bf16 MFMA.  Plant such values in a few tiles and bound every output element by the
    componentwise error of bf16 weights: |err| <= 2^-8 (|A_a| |V| + |lambda| |A_b| |V|) + 2^-8 |ref|.
    (Large planted values make O_a - lambda O_b cancel, so a row-RMS normalised check would be
    ill-conditioned here; an fp16 overflow or saturation of +-1e5 would exceed this bound by far.)"""
    log("v2 with |v| > 65504 in some tiles")
    N = 300
    t = wl.make_v2(1, 2, 1, N, 128, "bf16", seed=31, layers=(24,))
    vf = wl.as_f32(t["v"], "bf16").copy()
    vf[0, 0, 5, 7] = 1.0e5        # tile 0
    vf[0, 0, 130, 64] = -3.0e5    # tile 2
    vf[0, 0, 299, 127] = 7.0e4    # last, ragged tile
    t["v"] = wl.f32_to_bf16_bits(vf)
    got = _run_v2(da, t, 24, True)
    assert np.isfinite(got).all()
    ref = _oracle_v2(t, 24, True)
    lam = oracle_lambda(t["lambda"][24], 24)
    q, k, v = f64(t["q"]), f64(t["k"])[0, 0], f64(t["v"])[0, 0]
    worst = 0.0
    for p in range(2):
        a1, a2, _ = oracle.diff_maps(q[0, 2 * p], k, q[0, 2 * p + 1], k, lam[p], True)
        mag = np.abs(a1) @ np.abs(v) + abs(lam[p]) * (np.abs(a2) @ np.abs(v))
        err = np.abs(got[0, p] - ref[0, p])
        bound = 2.0 ** -8 * (mag + np.abs(ref[0, p]))
        worst = max(worst, float(np.max(err / bound)))
    log(f"  worst err / bound = {worst:.3f}")
    assert worst <= 1.0


def test_v2_workspace_contents_do_not_matter(da):
    """The V2 workspace (V rewritten as fp16 plus one flag byte per region) is clobbered by each
    call: a workspace full of garbage, one left by a call on other data (whose V tiles held values
    beyond the fp16 range, so its flags were set) and a fresh one give bit-identical outputs, for
    the causal and the windowed entry point."""
    import torch

    log("v2 workspace reuse")
    big = wl.make_v2(1, 2, 1, 300, 128, "bf16", seed=31, layers=(24,))
    vf = wl.as_f32(big["v"], "bf16").copy()
    vf[0, 0, ::7, ::5] = 1.0e5     # a value beyond fp16 in every 16-key x 64-channel region
    big["v"] = wl.f32_to_bf16_bits(vf)
    t = wl.make_v2(1, 2, 1, 257, 128, "bf16", seed=5, layers=(24,))
    need = max(da.diffattn_fwd_v2_workspace_bytes(1, 1, 300, 128),
               da.diffattn_fwd_v2_workspace_bytes(1, 1, 257, 128))
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    lv = dev_lambda(t["lambda"][24])
    first = {}
    for window in (0, 70):
        outs = []
        for fill in ("fresh", "garbage", "previous"):
            if fill == "fresh":
                ws = None
            elif fill == "garbage":
                ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
            else:
                ws = torch.zeros((need,), dtype=torch.uint8, device="cuda")
                qb = dev(big["q"])
                da.diffattn_fwd_v2(qb[:, 0::2], qb[:, 1::2], dev(big["k"]), dev(big["v"]),
                                   *dev_lambda(big["lambda"][24]), layer=24, workspace=ws)
            o = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], k, v, *lv, layer=24, window=window,
                                   workspace=ws)
            torch.cuda.synchronize()
            outs.append(o.cpu())
        assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]), window
        first[window] = outs[0]
    st = compare.bf16_stats(first[0].float().numpy(), _oracle_v2(t, 24, True), normalise=True)
    assert compare.bf16_ok(st), st


def test_v2_lambda_zero_is_even_heads_attention(da):
    """lambda = 0 gives plain softmax attention of the even query heads."""
    import torch

    log("v2 lambda override 0")
    t = wl.make_v2(1, 4, 2, 190, 128, "bf16", seed=77, layers=(24,))
    q = dev(t["q"])
    zero = torch.zeros(4, dtype=torch.float32, device="cuda")
    o = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], dev(t["k"]), dev(t["v"]), layer=24,
                           lambda_override=zero)
    torch.cuda.synchronize()
    ref = oracle.diff_attn_v2(f64(t["q"]), f64(t["k"]), f64(t["v"]), np.zeros(4), True)
    st = compare.bf16_stats(o.float().cpu().numpy(), ref, normalise=True)
    assert compare.bf16_ok(st), st


@pytest.mark.timeout(600)
def test_v2_workload_8k_every_pair(da):
    """Full V2 prefill workload (B=2, 32 query heads / 16 pairs over 8 KV heads, D=128, N=8192,
    causal, l=24): 2048 rows (the first and last 64 among them) of every (batch, pair)."""
    import torch

    cfg, t = wl.make("v2_prefill_8k")
    layer = cfg["layers"][0]
    B, P, Hkv, N = cfg["B"], cfg["P"], cfg["Hkv"], cfg["N"]
    log("v2 B=2 P=16 Hkv=8 N=8192 (full launch, 2048 rows of every pair)")
    lam_out = torch.full((P,), float("nan"), dtype=torch.float32, device="cuda")
    got = _run_v2(da, t, layer, lambda_out=lam_out)
    assert np.isfinite(got).all()
    lam = oracle_lambda(t["lambda"][layer], layer)
    np.testing.assert_allclose(lam_out.cpu().numpy(), lam, rtol=0, atol=2e-6)
    rows = sample_rows(N, 2048 - 128, seed=3, extra=tuple(range(64)) + tuple(range(N - 64, N)))

    def one(bp):
        b, p = divmod(bp, P)
        g = p * Hkv // P
        q = f64(t["q"][b:b + 1, 2 * p:2 * p + 2])
        ref = oracle.diff_attn_v2(q, f64(t["k"][b:b + 1, g:g + 1]), f64(t["v"][b:b + 1, g:g + 1]),
                                  lam[p:p + 1], True, rows=rows)[0, 0]
        return b, p, compare.bf16_stats(got[b, p, rows], ref, normalise=True)

    worst = None
    for b, p, st in parallel_map(one, range(B * P)):
        assert compare.bf16_ok(st), (b, p, st)
        worst = st if worst is None or st["max_abs"] > worst["max_abs"] else worst
    log(f"  {B * P} pairs x {rows.size} rows ok, worst {worst}")

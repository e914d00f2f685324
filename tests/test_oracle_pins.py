"""Pins of the float64 CPU oracle against things other than itself.

Each test checks the oracle against values the source pages print, closed forms that follow from
the pages' definitions, special cases that reduce to a library routine (torch's float64 SDPA and
rms_norm on the CPU), invariants of softmax, or the independent pure-Python brute force.  They are
chosen so that a plausible slip in the oracle -- a dropped term, a wrong sign, a transposed
operand, the wrong width under the square root, the wrong lambda in the scale -- fails at least
one of them (``test_mutations_are_caught`` plants such slips and checks exactly that).

Sources: [G] Ultralytics glossary "Differential Transformer", section "Cómo funciona la atención
diferencial"; [L] ai-engineering.academy "Atención Diferencial (V2)", sections "La idea
diferencial", "V1 vs V2: la diferencia", "Implementación", "Ejercicios".
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import bruteforce as bfm
from oracle import diffattn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            vals[k] = v
    return vals


def _rng(seed):
    return np.random.default_rng(seed)


def _heads(rng, B, H, N, d, dv):
    q1, q2, k1, k2 = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    v = rng.standard_normal((B, H, N, dv))
    return q1, q2, k1, k2, v


def _sdpa(q, k, v, causal):
    """torch float64 CPU scaled-dot-product attention (default scale 1/sqrt(q width))."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal).numpy()


# ------------------------------------------------------------------------------------------------
# values printed by the pages
# ------------------------------------------------------------------------------------------------

def test_worked_example_printed_values():
    """[G] worked example: seed 0, n=6, d=8, lambda=0.8 prints row sum 0.20 and 13 of 36 negative."""
    g = _golden("worked_example.txt")
    n, d, lam = int(g["n"]), int(g["d"]), float(g["lambda"])
    torch.manual_seed(int(g["seed"]))
    q1, k1, q2, k2 = torch.randn(4, n, d)
    _v = torch.randn(n, 2 * d)  # drawn to keep the generator in the page's order
    a1, a2, w = oracle.diff_maps(q1.numpy(), k1.numpy(), q2.numpy(), k2.numpy(), lam)
    assert f"{w.sum(axis=-1)[0]:.2f}" == g["row0_sum_2dp"]
    assert int((w < 0).sum()) == int(g["negative_weights"])
    assert w.size == int(g["total_weights"])
    # the count is robust: no weight sits within rounding distance of zero
    assert np.min(np.abs(w)) > 1e-4


def test_lambda_init_schedule_special_values():
    g = _golden("lambda_init_schedule.txt")
    assert oracle.lambda_init(1) == pytest.approx(float(g["layer1"]), abs=1e-15)
    vals = [oracle.lambda_init(l) for l in range(1, 64)]
    assert all(b > a for a, b in zip(vals, vals[1:]))          # deeper layers start higher
    assert all(v < float(g["asymptote"]) for v in vals)
    assert oracle.lambda_init(400) == pytest.approx(float(g["asymptote"]), abs=1e-15)
    # the gap to 0.8 loses digits to cancellation in deep layers, so check the ratio early on
    gaps = [float(g["asymptote"]) - v for v in vals[:20]]
    for a, b in zip(gaps, gaps[1:]):
        assert math.log(b / a) == pytest.approx(float(g["gap_ratio_log"]), abs=1e-8)
    with pytest.raises(ValueError):
        oracle.lambda_init(0)


# ------------------------------------------------------------------------------------------------
# lambda parameterisation ([L] "La idea diferencial")
# ------------------------------------------------------------------------------------------------

def test_lambda_zero_vectors_give_lambda_init():
    z = np.zeros((3, 64))
    for l in (1, 5, 24):
        np.testing.assert_array_equal(oracle.lambda_value(z, z, z, z, l),
                                      np.full(3, oracle.lambda_init(l)))


def test_lambda_closed_form_single_coordinate():
    d = 16
    for a in (-1.3, 0.0, 0.4, 2.0):
        lq1 = np.zeros((1, d)); lq1[0, 0] = a
        lk1 = np.zeros((1, d)); lk1[0, 0] = 1.0
        z = np.zeros((1, d))
        lam = oracle.lambda_value(lq1, lk1, z, z, 3)[0]
        assert lam == pytest.approx(math.e ** a - 1.0 + oracle.lambda_init(3), abs=1e-14)
        # moving the same vectors to the second pair flips the sign of the learned part
        lam2 = oracle.lambda_value(z, z, lq1, lk1, 3)[0]
        assert lam2 - oracle.lambda_init(3) == pytest.approx(-(lam - oracle.lambda_init(3)), abs=1e-14)


def test_lambda_can_be_negative_and_above_one():
    d = 4
    big = np.zeros((1, d)); big[0, 0] = 2.0
    one = np.zeros((1, d)); one[0, 0] = 1.0
    z = np.zeros((1, d))
    assert oracle.lambda_value(z, z, big, one, 1)[0] < 0      # not clamped below
    assert oracle.lambda_value(big, one, z, z, 1)[0] > 1      # not clamped above


# ------------------------------------------------------------------------------------------------
# maps and their difference ([G], [L])
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_difference_rows_sum_to_one_minus_lambda(causal):
    rng = _rng(1)
    q1, q2, k1, k2, _ = (a[0, 0] for a in _heads(rng, 1, 1, 37, 8, 16))
    for lam in (0.8, -0.3, 1.7):
        a1, a2, w = oracle.diff_maps(q1, k1, q2, k2, lam, causal)
        np.testing.assert_allclose(a1.sum(-1), 1.0, atol=1e-13)
        np.testing.assert_allclose(a2.sum(-1), 1.0, atol=1e-13)
        np.testing.assert_allclose(w.sum(-1), 1.0 - lam, atol=1e-12)
        assert np.all(a1 >= 0) and np.all(a2 >= 0)
    _, _, w = oracle.diff_maps(q1, k1, q2, k2, 0.8, causal)
    assert (w < 0).sum() > 0                                    # negative weights appear
    if causal:
        assert np.all(np.triu(w, 1) == 0)                      # future keys carry exactly 0


@pytest.mark.parametrize("causal", [False, True])
def test_lambda_zero_is_standard_attention_v1(causal):
    """[L] "Ejercicios" 4: lambda = 0 leaves the first softmax branch alone -> library SDPA."""
    rng = _rng(2)
    q1, q2, k1, k2, v = _heads(rng, 2, 3, 29, 64, 128)
    got = oracle.diff_attn_v1(q1, q2, k1, k2, v, np.zeros(3), 0.2, causal, norm=False)
    ref = _sdpa(q1, k1, v, causal)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_branches_full_subtraction_is_zero(causal):
    """[L] "Ejercicios" 4, lambda = 1 with both branches equal: the difference map vanishes."""
    rng = _rng(3)
    q, _, k, _, v = _heads(rng, 1, 2, 21, 64, 128)
    core = oracle.diff_attn_v1(q, q, k, k, v, np.ones(2), 0.2, causal, norm=False)
    assert np.max(np.abs(core)) < 1e-13
    y = oracle.diff_attn_v1(q, q, k, k, v, np.ones(2), 0.2, causal, eps=1e-5)
    assert np.max(np.abs(y)) < 1e-10                            # |y| <= |O| / sqrt(eps)


@pytest.mark.parametrize("causal", [False, True])
def test_general_lambda_against_two_library_sdpa_calls(causal):
    rng = _rng(4)
    q1, q2, k1, k2, v = _heads(rng, 1, 4, 33, 64, 128)
    lam = np.array([0.8, -0.4, 1.3, 0.05])
    got = oracle.diff_attn_v1(q1, q2, k1, k2, v, lam, 0.5, causal, norm=False)
    ref = _sdpa(q1, k1, v, causal) - lam[None, :, None, None] * _sdpa(q2, k2, v, causal)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_key_shift_invariance():
    """Adding one vector to every key of a branch shifts each score row by a constant."""
    rng = _rng(5)
    q1, q2, k1, k2, v = (a[0, 0] for a in _heads(rng, 1, 1, 25, 16, 32))
    u1, u2 = rng.standard_normal(16), rng.standard_normal(16)
    for causal in (False, True):
        base = oracle.diff_core_rows(q1, k1, q2, k2, v, 0.7, causal)
        shifted = oracle.diff_core_rows(q1, k1 + u1, q2, k2 + u2, v, 0.7, causal)
        np.testing.assert_allclose(shifted, base, atol=1e-11)


def test_joint_key_value_permutation_invariance_noncausal():
    rng = _rng(6)
    q1, q2, k1, k2, v = (a[0, 0] for a in _heads(rng, 1, 1, 19, 16, 32))
    perm = rng.permutation(19)
    base = oracle.diff_core_rows(q1, k1, q2, k2, v, 0.6, False)
    perm_out = oracle.diff_core_rows(q1, k1[perm], q2, k2[perm], v[perm], 0.6, False)
    np.testing.assert_allclose(perm_out, base, atol=1e-12)


def test_causal_first_row_and_uniform_maps():
    rng = _rng(7)
    _, _, k1, k2, v = (a[0, 0] for a in _heads(rng, 1, 1, 23, 16, 32))
    q0 = np.zeros((23, 16))
    lam = 0.35
    out = oracle.diff_core_rows(q0, k1, q0, k2, v, lam, True)
    # zero queries give uniform maps over the visible keys
    ref = (1 - lam) * np.cumsum(v, axis=0) / np.arange(1, 24)[:, None]
    np.testing.assert_allclose(out, ref, atol=1e-13)
    q1, q2 = rng.standard_normal((23, 16)), rng.standard_normal((23, 16))
    out = oracle.diff_core_rows(q1, k1, q2, k2, v, lam, True)
    np.testing.assert_allclose(out[0], (1 - lam) * v[0], atol=1e-14)


def test_scale_uses_branch_width():
    """The square root is of the per-branch width (the worked example divides by sqrt(8) with
    halves of width 8): a width-d branch equals SDPA with its default 1/sqrt(d) scale, not a
    1/sqrt(2d) one."""
    rng = _rng(8)
    q1, q2, k1, k2, v = _heads(rng, 1, 1, 17, 8, 16)
    got = oracle.diff_attn_v1(q1, q2, k1, k2, v, np.zeros(1), 0.2, False, norm=False)
    wrong = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q1, k1, v)),
                                           scale=1 / math.sqrt(16)).numpy()
    assert np.max(np.abs(got - wrong)) > 1e-3
    np.testing.assert_allclose(got, _sdpa(q1, k1, v, False), atol=1e-12)


# ------------------------------------------------------------------------------------------------
# per-head normalisation and scale ([G])
# ------------------------------------------------------------------------------------------------

def test_rms_norm_matches_library_routine():
    rng = _rng(9)
    o = rng.standard_normal((7, 128)) * 0.03
    ref = F.rms_norm(torch.from_numpy(o), (128,), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm_rows(o, 1e-5), ref, rtol=1e-13, atol=1e-15)


def test_v1_output_rms_and_scale_uses_lambda_init():
    rng = _rng(10)
    q1, q2, k1, k2, v = _heads(rng, 1, 2, 31, 64, 128)
    lam = np.array([0.9, 0.3])     # learned lambdas differ from lambda_init on purpose
    lam_init = oracle.lambda_init(12)
    eps = 1e-5
    y = oracle.diff_attn_v1(q1, q2, k1, k2, v, lam, lam_init, True, eps)
    core = oracle.diff_attn_v1(q1, q2, k1, k2, v, lam, lam_init, True, eps, norm=False)
    ms = np.mean(core ** 2, axis=-1)
    rms_y = np.sqrt(np.mean(y ** 2, axis=-1))
    np.testing.assert_allclose(rms_y, (1 - lam_init) * np.sqrt(ms / (ms + eps)), rtol=1e-12)
    ref = F.rms_norm(torch.from_numpy(core), (128,), eps=eps).numpy() * (1 - lam_init)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------------------------------------
# V2 layout and decode ([L] "V1 vs V2: la diferencia", "Ejercicios" 5)
# ------------------------------------------------------------------------------------------------

def _gqa_sdpa(q_heads, k, v, causal):
    """Baseline GQA through torch SDPA: query head h reads KV head h // (Hq / Hkv)."""
    rep = q_heads.shape[1] // k.shape[1]
    kk = np.repeat(k, rep, axis=1)
    vv = np.repeat(v, rep, axis=1)
    return _sdpa(q_heads, kk, vv, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_v2_against_library_gqa(causal):
    rng = _rng(11)
    B, P, Hkv, N, D = 2, 8, 2, 19, 32
    q = rng.standard_normal((B, 2 * P, N, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    lam = rng.uniform(-0.5, 1.5, P)
    got = oracle.diff_attn_v2(q, k, v, lam, causal)
    base = _gqa_sdpa(q, k, v, causal)                       # baseline GQA over all 2P heads
    ref = base[:, 0::2] - lam[None, :, None, None] * base[:, 1::2]
    np.testing.assert_allclose(got, ref, atol=1e-12)
    # lambda = 0: the even heads alone
    np.testing.assert_allclose(oracle.diff_attn_v2(q, k, v, np.zeros(P), causal), base[:, 0::2],
                               atol=1e-12)


def test_v2_kv_cache_matches_baseline_gqa_size():
    """[L] "Ejercicios" 5: with 32 query heads over 8 KV heads the V2 cache is the GQA(8, 32) one."""
    B, L, D = 3, 100, 128
    hq, hkv = 32, 8
    P = hq // 2
    q = np.zeros((B, hq, D)); k = np.zeros((B, hkv, L, D)); v = np.zeros((B, hkv, L, D))
    out = oracle.diff_decode_v2(q, k, v, np.zeros(P))
    assert k.nbytes + v.nbytes == 2 * B * hkv * L * D * 8
    assert out.shape == (B, P, D)


def test_v2_with_shared_keys_equals_v1_bookkeeping():
    """[L] "Implementación" step 2: V1 and V2 are the same mathematics with different layouts."""
    rng = _rng(12)
    N, d = 15, 16
    q1, q2, k, v = (rng.standard_normal((1, 1, N, w)) for w in (d, d, d, 2 * d))
    lam = np.array([0.7])
    v1 = oracle.diff_attn_v1(q1, q2, k, k, v, lam, 0.2, True, norm=False)
    q = np.concatenate([q1, q2], axis=1)            # heads (0, 1) form pair 0
    v2 = oracle.diff_attn_v2(q, k, v, lam, True)
    np.testing.assert_allclose(v2, v1, atol=1e-13)


def test_decode_is_last_prefill_row():
    rng = _rng(13)
    B, P, Hkv, L, D = 2, 4, 2, 27, 16
    q = rng.standard_normal((B, 2 * P, L, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    lam = rng.uniform(0, 1, P)
    pre = oracle.diff_attn_v2(q, k, v, lam, True)
    dec = oracle.diff_decode_v2(q[:, :, -1], k, v, lam)
    np.testing.assert_allclose(dec, pre[:, :, -1], atol=1e-13)
    # V1 decode likewise
    q1, q2, k1, k2, vv = _heads(rng, 2, 3, L, 8, 16)
    lam1 = np.array([0.1, 0.8, 1.2])
    pre1 = oracle.diff_attn_v1(q1, q2, k1, k2, vv, lam1, 0.4, True)
    dec1 = oracle.diff_decode_v1(q1[:, :, -1], q2[:, :, -1], k1, k2, vv, lam1, 0.4)
    np.testing.assert_allclose(dec1, pre1[:, :, -1], atol=1e-12)


# ------------------------------------------------------------------------------------------------
# brute force and sampled evaluation
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 7, 16])
def test_brute_force_agreement_v1(n, causal):
    rng = _rng(100 + n)
    d = 8
    q1, q2, k1, k2, v = (a[0, 0] for a in _heads(rng, 1, 1, n, d, 2 * d))
    lvec = [rng.standard_normal(d) * 0.1 for _ in range(4)]
    layer = 1 + n % 5
    lam_bf = bfm.head_lambda(*(x.tolist() for x in lvec), layer)
    lam = oracle.lambda_value(*(x[None] for x in lvec), layer)[0]
    assert lam == pytest.approx(lam_bf, abs=1e-14)
    lam_init = oracle.lambda_init(layer)
    ref = bfm.v1_head(q1.tolist(), k1.tolist(), q2.tolist(), k2.tolist(), v.tolist(), lam_bf,
                      bfm.layer_lambda_init(layer), causal, 1e-5)
    got = oracle.diff_attn_v1(q1[None, None], q2[None, None], k1[None, None], k2[None, None],
                              v[None, None], np.array([lam]), lam_init, causal, 1e-5)[0, 0]
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_agreement_v2(causal):
    rng = _rng(200)
    N, D = 11, 8
    qa, qb, k, v = (rng.standard_normal((N, D)) for _ in range(4))
    ref = bfm.v2_pair(qa.tolist(), qb.tolist(), k.tolist(), v.tolist(), 0.6, causal)
    q = np.stack([qa, qb])[None]
    got = oracle.diff_attn_v2(q, k[None, None], v[None, None], np.array([0.6]), causal)[0, 0]
    np.testing.assert_allclose(got, np.array(ref), atol=1e-12)


def test_sampled_rows_equal_full_rows():
    rng = _rng(14)
    q1, q2, k1, k2, v = _heads(rng, 1, 2, 300, 16, 32)
    full = oracle.diff_attn_v1(q1, q2, k1, k2, v, np.array([0.2, 0.9]), 0.3, True)
    rows = [0, 5, 133, 299]
    part = oracle.diff_attn_v1(q1, q2, k1, k2, v, np.array([0.2, 0.9]), 0.3, True, rows=rows,
                               heads=[1])
    np.testing.assert_allclose(part[0, 0], full[0, 1, rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5)])
def test_layer_sweep_equals_per_layer_v1(causal, window):
    """The layer-sweep entry (branch outputs formed once, lambda applied per layer) equals the
    plain V1 definition evaluated layer by layer, for every head, row and layer."""
    rng = _rng(16)
    q1, q2, k1, k2, v = _heads(rng, 2, 3, 37, 8, 16)
    layers = [1, 2, 7, 32]
    lams = np.array([rng.uniform(-0.6, 1.6, 3) for _ in layers])
    inits = [oracle.lambda_init(l) for l in layers]
    rows = [0, 3, 17, 36]
    got = oracle.diff_attn_v1_layers(q1, q2, k1, k2, v, lams, inits, causal, 1e-5, rows=rows,
                                     heads=[0, 2], window=window)
    for li in range(len(layers)):
        ref = oracle.diff_attn_v1(q1, q2, k1, k2, v, lams[li], inits[li], causal, 1e-5, rows=rows,
                                  heads=[0, 2], window=window)
        np.testing.assert_allclose(got[li], ref, rtol=0, atol=1e-12)
    # a lambda taken from the wrong layer or head, or the wrong lambda_init, is visible
    bad = oracle.diff_attn_v1_layers(q1, q2, k1, k2, v, lams[::-1], inits, causal, 1e-5, rows=rows,
                                     heads=[0, 2], window=window)
    assert np.max(np.abs(bad - got)) > 1e-3
    bad = oracle.diff_attn_v1_layers(q1, q2, k1, k2, v, lams, inits[::-1], causal, 1e-5, rows=rows,
                                     heads=[0, 2], window=window)
    assert np.max(np.abs(bad - got)) > 1e-3
    with pytest.raises(ValueError):
        oracle.diff_attn_v1_layers(q1, q2, k1, k2, v, lams[:, :2], inits, causal)


def test_row_blocking_does_not_change_values(monkeypatch):
    rng = _rng(15)
    q1, q2, k1, k2, v = (a[0, 0] for a in _heads(rng, 1, 1, 90, 16, 32))
    a = oracle.diff_core_rows(q1, k1, q2, k2, v, 0.5, True)
    monkeypatch.setattr(orc, "_MAX_BLOCK_ENTRIES", 200)   # many small row blocks
    b = oracle.diff_core_rows(q1, k1, q2, k2, v, 0.5, True)
    np.testing.assert_allclose(a, b, atol=1e-14)


# ------------------------------------------------------------------------------------------------
# planted mistakes: each plausible slip must fail at least one pin above
# ------------------------------------------------------------------------------------------------

def _mutant_core(kind):
    def core(q1, k1, q2, k2, v, lam, causal, rows=None, window=0):
        q1, k1, q2, k2, v = (np.asarray(a, dtype=np.float64) for a in (q1, k1, q2, k2, v))
        d = q1.shape[-1]
        n = q1.shape[0]
        rows_ = np.arange(n) if rows is None else np.asarray(rows)
        vis = (np.arange(k1.shape[0])[None, :] <= rows_[:, None]) if causal else None
        scale = math.sqrt(2 * d) if kind == "wide_scale" else math.sqrt(d)
        s1 = q1[rows_] @ k1.T / scale
        s2 = q2[rows_] @ k2.T / scale
        if kind == "transposed":
            s1 = (k1 @ q1.T / scale)[rows_]
        a1 = orc.softmax_rows(s1, vis)
        a2 = orc.softmax_rows(s2, vis)
        if kind == "plus_sign":
            return (a1 + lam * a2) @ v
        if kind == "dropped_branch":
            return a1 @ v
        if kind == "swapped_branch_keys":
            return (orc.softmax_rows(q1[rows_] @ k2.T / scale, vis) - lam * a2) @ v
        return (a1 - lam * a2) @ v
    return core


PINS_FOR_CORE = [
    test_general_lambda_against_two_library_sdpa_calls,
    test_lambda_zero_is_standard_attention_v1,
    test_scale_uses_branch_width,
    test_difference_rows_sum_to_one_minus_lambda,
]


@pytest.mark.parametrize("kind", ["plus_sign", "dropped_branch", "wide_scale", "transposed",
                                  "swapped_branch_keys"])
def test_mutations_are_caught(kind, monkeypatch):
    monkeypatch.setattr(orc, "diff_core_rows", _mutant_core(kind))
    failed = 0
    for pin in PINS_FOR_CORE:
        for causal in (False, True):
            try:
                if pin is test_scale_uses_branch_width:
                    pin()
                else:
                    pin(causal)
            except AssertionError:
                failed += 1
    assert failed > 0, f"mutation {kind!r} slipped through every pin"


def test_mutated_scale_in_v1_is_caught(monkeypatch):
    """Scaling by (1 - lambda) instead of (1 - lambda_init) must fail the RMS/scale pin."""
    real = orc.diff_attn_v1

    def mutant(q1, q2, k1, k2, v, lam, lam_init, causal=True, eps=1e-5, norm=True, **kw):
        out = real(q1, q2, k1, k2, v, lam, lam_init, causal, eps, norm=False, **kw)
        if norm:
            lam_b = np.broadcast_to(np.asarray(lam, dtype=np.float64), (q1.shape[1],))
            out = orc.rms_norm_rows(out, eps) * (1 - lam_b)[None, :, None, None]
        return out

    monkeypatch.setattr(oracle, "diff_attn_v1", mutant)
    with pytest.raises(AssertionError):
        test_v1_output_rms_and_scale_uses_lambda_init()


# ------------------------------------------------------------------------------------------------
# sliding window (causal; row i sees its last W positions)
# ------------------------------------------------------------------------------------------------

def _band(n, window):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return torch.from_numpy((j <= i) & (j > i - window))


def test_window_against_library_sdpa_with_band_mask():
    """Both branches as library SDPA calls restricted by an explicit band mask."""
    rng = _rng(31)
    q1, q2, k1, k2, v = _heads(rng, 1, 3, 40, 64, 128)
    lam = np.array([0.7, -0.2, 1.1])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    for window in (1, 3, 17, 39, 40, 64):
        m = _band(40, window)
        ref = (F.scaled_dot_product_attention(t(q1), t(k1), t(v), attn_mask=m).numpy()
               - lam[None, :, None, None] * F.scaled_dot_product_attention(t(q2), t(k2), t(v), attn_mask=m).numpy())
        got = oracle.diff_attn_v1(q1, q2, k1, k2, v, lam, 0.5, True, norm=False, window=window)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_of_one_sees_only_itself():
    """W = 1: both maps are the identity, so the core is (1 - lambda) V row by row."""
    rng = _rng(32)
    q1, q2, k1, k2, v = _heads(rng, 1, 2, 25, 64, 128)
    lam = np.array([0.3, 1.4])
    got = oracle.diff_attn_v1(q1, q2, k1, k2, v, lam, 0.5, True, norm=False, window=1)
    np.testing.assert_allclose(got, (1 - lam)[None, :, None, None] * v, rtol=0, atol=1e-13)
    qv = np.concatenate([q1, q2], axis=1)
    g2 = oracle.diff_attn_v2(qv[:, [0, 2, 1, 3]], k1[:, :1], v[:, :1], lam, True, window=1)
    np.testing.assert_allclose(g2, (1 - lam)[None, :, None, None] * v[:, :1], rtol=0, atol=1e-13)


def test_window_covering_every_row_is_plain_causal():
    rng = _rng(33)
    q1, q2, k1, k2, v = _heads(rng, 1, 2, 30, 16, 32)
    a = oracle.diff_attn_v1(q1, q2, k1, k2, v, np.array([0.4, 0.6]), 0.5, True)
    for window in (30, 31, 1000):
        b = oracle.diff_attn_v1(q1, q2, k1, k2, v, np.array([0.4, 0.6]), 0.5, True, window=window)
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("n", [1, 6, 13])
def test_window_brute_force_agreement(n):
    rng = _rng(300 + n)
    d = 8
    q1, q2, k1, k2, v = (a[0, 0] for a in _heads(rng, 1, 1, n, d, 2 * d))
    for window in range(1, n + 2):
        ref = bfm.diff_attention(q1.tolist(), k1.tolist(), q2.tolist(), k2.tolist(), v.tolist(),
                                 0.7, True, window)
        got = oracle.diff_core_rows(q1, k1, q2, k2, v, 0.7, True, window=window)
        np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=1e-12)
        refb = bfm.attention(q1.tolist(), k1.tolist(), v.tolist(), True, window)
        gotb = oracle.branch_rows(q1, k1, v, True, window=window)
        np.testing.assert_allclose(gotb, np.array(refb), rtol=0, atol=1e-12)


def test_window_requires_causal():
    rng = _rng(34)
    q1, q2, k1, k2, v = _heads(rng, 1, 1, 8, 8, 16)
    with pytest.raises(ValueError):
        oracle.diff_attn_v1(q1, q2, k1, k2, v, np.array([0.5]), 0.5, False, window=4)


@pytest.mark.parametrize("kind", ["off_by_one_wide", "off_by_one_narrow"])
def test_window_mutations_are_caught(kind, monkeypatch):
    real = orc._visible

    def mutant(rows, n_keys, causal, window=0):
        if not window:
            return real(rows, n_keys, causal, window)
        keys = np.arange(n_keys)
        vis = keys[None, :] <= rows[:, None]
        lo = rows[:, None] - window + (-1 if kind == "off_by_one_wide" else 1)
        return vis & (keys[None, :] > lo)

    monkeypatch.setattr(orc, "_visible", mutant)
    caught = 0
    for pin in (test_window_against_library_sdpa_with_band_mask, test_window_of_one_sees_only_itself):
        try:
            pin()
        except (AssertionError, ValueError):  # a wrong value, or a row left with no key
            caught += 1
    assert caught > 0, f"window mutation {kind!r} slipped through"

"""CPU pins of the float64 backward oracle (``oracle.diff_attn_v1_backward``).

Its gradients are checked against two derivations that share nothing with it: torch float64
autograd through the forward definition written with library ops, and central finite
differences of the numpy forward oracle.  Perturbed gradients (sign, transposition, small
offsets) must fail the autograd pin, which shows its sensitivity.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import diffattn_backward as bwd


def _inputs(seed, B=1, H=2, N=9, d=8, dl=8):
    rng = np.random.default_rng(seed)
    q1, q2, k1, k2 = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    v = rng.standard_normal((B, H, N, 2 * d))
    dy = rng.standard_normal((B, H, N, 2 * d))
    lv = tuple(rng.standard_normal((H, dl)) * 0.3 for _ in range(4))
    return q1, q2, k1, k2, v, dy, lv


def _torch_forward(q1, q2, k1, k2, v, lv, layer, causal, eps, window=0):
    """The V1 forward with torch ops (differentiated by autograd)."""
    d = q1.shape[-1]
    n = q1.shape[-2]
    mask = None
    if causal:
        i = torch.arange(n)[:, None]
        j = torch.arange(n)[None, :]
        mask = j <= i
        if window:
            mask = mask & (j > i - window)
    lam = (torch.exp((lv[0] * lv[1]).sum(-1)) - torch.exp((lv[2] * lv[3]).sum(-1))
           + (0.8 - 0.6 * math.exp(-0.3 * (layer - 1))))
    def amap(q, k):
        s = q @ k.transpose(-1, -2) / math.sqrt(d)
        if mask is not None:
            s = s.masked_fill(~mask, float("-inf"))
        return torch.softmax(s, dim=-1)
    o = amap(q1, k1) @ v - lam[None, :, None, None] * (amap(q2, k2) @ v)
    y = o / torch.sqrt((o * o).mean(-1, keepdim=True) + eps)
    return y * (1 - (0.8 - 0.6 * math.exp(-0.3 * (layer - 1))))


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 3)])
def test_backward_matches_autograd(causal, window):
    q1, q2, k1, k2, v, dy, lv = _inputs(1)
    layer = 4
    got = oracle.diff_attn_v1_backward(q1, q2, k1, k2, v, lv, layer, dy, causal, 1e-5, window)
    ts = [torch.tensor(x, requires_grad=True) for x in (q1, q2, k1, k2, v)]
    tl = [torch.tensor(x, requires_grad=True) for x in lv]
    y = _torch_forward(*ts, tl, layer, causal, 1e-5, window)
    (y * torch.tensor(dy)).sum().backward()
    for name, t in zip(("dq1", "dq2", "dk1", "dk2", "dv"), ts):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)
    for name, t in zip(("dlq1", "dlk1", "dlq2", "dlk2"), tl):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)


def test_backward_matches_finite_differences():
    """Central differences of the numpy forward oracle on a few coordinates of every input."""
    q1, q2, k1, k2, v, dy, lv = _inputs(2, H=1, N=6, d=4, dl=4)
    layer, eps, h = 3, 1e-5, 1e-5
    grads = oracle.diff_attn_v1_backward(q1, q2, k1, k2, v, lv, layer, dy, True, eps)

    def loss(arrs, lvs):
        lam = oracle.lambda_value(*lvs, layer)
        y = oracle.diff_attn_v1(*arrs, lam, oracle.lambda_init(layer), True, eps)
        return float(np.sum(y * dy))

    arrs = [q1, q2, k1, k2, v]
    names = ["dq1", "dq2", "dk1", "dk2", "dv"]
    rng = np.random.default_rng(0)
    for ai, name in enumerate(names):
        for _ in range(4):
            idx = tuple(rng.integers(0, s) for s in arrs[ai].shape)
            plus = [a.copy() for a in arrs]
            minus = [a.copy() for a in arrs]
            plus[ai][idx] += h
            minus[ai][idx] -= h
            fd = (loss(plus, lv) - loss(minus, lv)) / (2 * h)
            assert grads[name][idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, idx)
    for li, name in enumerate(["dlq1", "dlk1", "dlq2", "dlk2"]):
        idx = (0, int(rng.integers(0, 4)))
        plus = [x.copy() for x in lv]
        minus = [x.copy() for x in lv]
        plus[li][idx] += h
        minus[li][idx] -= h
        fd = (loss(arrs, plus) - loss(arrs, minus)) / (2 * h)
        assert grads[name][idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), name


def test_zero_upstream_gradient_gives_zero():
    q1, q2, k1, k2, v, dy, lv = _inputs(3)
    got = oracle.diff_attn_v1_backward(q1, q2, k1, k2, v, lv, 2, np.zeros_like(dy))
    for k, x in got.items():
        assert np.all(x == 0), k


@pytest.mark.parametrize("slip", ["softmax_rowsum", "dv_sign", "norm_term", "dk_transpose"])
def test_backward_slips_are_caught(slip, monkeypatch):
    """Perturb one gradient the way a chain-rule slip would and check the autograd pin fails."""
    real = bwd.diff_attn_v1_backward

    def mutant(q1, q2, k1, k2, v, lvecs, layer, dy, causal=True, eps=1e-5, window=0):
        out = real(q1, q2, k1, k2, v, lvecs, layer, dy, causal, eps, window)
        if slip == "softmax_rowsum":        # a small bias like a dropped Jacobian term
            out["dq1"] = out["dq1"] + 1e-3 * np.sign(out["dq1"])
        elif slip == "dv_sign":             # + lam A2^T dO instead of -
            out["dv"] = -out["dv"]
        elif slip == "norm_term":           # a 1 % scale error in a lambda gradient
            out["dlq1"] = out["dlq1"] * 1.01
        elif slip == "dk_transpose":
            out["dk2"] = out["dk2"][..., ::-1, :]
        return out

    monkeypatch.setattr(oracle, "diff_attn_v1_backward", mutant)
    with pytest.raises(AssertionError):
        test_backward_matches_autograd(True, 0)

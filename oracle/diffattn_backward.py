"""Plain float64 CPU oracle of the V1 differential-attention BACKWARD pass.

TEST INFRASTRUCTURE ONLY (same rules as ``diffattn_oracle``): imported by ``tests/`` and
``bench.py``'s CPU baseline, never by the product path, and shares no code with the HIP library.

It differentiates the forward definition ([G] Ultralytics glossary "Differential Transformer",
section "Cómo funciona la atención diferencial"; [L] ai-engineering.academy "Atención
Diferencial (V2)", section "La idea diferencial") by the chain rule, one head at a time, on
whole [N, N] maps -- no tiling, no recomputation tricks:

  forward   S_b = Q_b K_b^T c  (c = 1 / sqrt(d)),  A_b = softmax(S_b) (row-wise, causal mask),
            O_b = A_b V,  O = O_1 - lam O_2,
            r = (mean(O^2) + eps)^(-1/2) per row,  y = g r O  with g = 1 - lambda_init,
            lam = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lambda_init.
  backward  dO = g r dy - g r^3 (O . dy) O / n                 (RMS norm, n = 2d channels)
            dV = A_1^T dO - lam A_2^T dO
            dA_1 = dO V^T,  dA_2 = -lam dO V^T
            dS_b = A_b * (dA_b - rowsum(A_b * dA_b))           (softmax Jacobian)
            dQ_b = c dS_b K_b,  dK_b = c dS_b^T Q_b
            dlam = -sum(dO * O_2) over the head's rows (and batch)
            dlq1 = dlam e^<lq1,lk1> lk1,  dlk1 = dlam e^<lq1,lk1> lq1,
            dlq2 = -dlam e^<lq2,lk2> lk2, dlk2 = -dlam e^<lq2,lk2> lq2.
"""

from __future__ import annotations

import math

import numpy as np

from .diffattn_oracle import lambda_init, softmax_rows

__all__ = ["diff_attn_v1_backward"]


def _mask(n: int, causal: bool, window: int):
    if not causal:
        return None
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = j <= i
    if window:
        vis &= j > i - window
    return vis


def diff_attn_v1_backward(q1, q2, k1, k2, v, lvecs, layer: int, dy, causal: bool = True,
                          eps: float = 1e-5, window: int = 0):
    """Gradients of the V1 output y [B, H, N, 2d] with respect to every input, given dy.

    q1, q2, k1, k2 [B, H, N, d]; v, dy [B, H, N, 2d]; lvecs = (lq1, lk1, lq2, lk2), each [H, dl].
    Returns a dict with dq1, dq2, dk1, dk2, dv (input shapes), dlam [H] and dlq1, dlk1, dlq2,
    dlk2 ([H, dl]), all float64, and dlam_terms [H] = sum over rows and channels of |dO * O_2|,
    the magnitude of dlam's terms before they cancel (an error scale for comparisons).
    """
    q1, q2, k1, k2, v, dy = (np.asarray(a, dtype=np.float64) for a in (q1, q2, k1, k2, v, dy))
    lq1, lk1, lq2, lk2 = (np.asarray(a, dtype=np.float64) for a in lvecs)
    B, H, N, d = q1.shape
    n = v.shape[-1]
    c = 1.0 / math.sqrt(d)
    li = lambda_init(layer)
    g = 1.0 - li
    ea = np.exp(np.sum(lq1 * lk1, axis=-1))
    eb = np.exp(np.sum(lq2 * lk2, axis=-1))
    lam = ea - eb + li
    vis = _mask(N, causal, window)
    out = {k: np.zeros_like(x) for k, x in (("dq1", q1), ("dq2", q2), ("dk1", k1), ("dk2", k2),
                                            ("dv", v))}
    dlam = np.zeros(H)
    dlam_terms = np.zeros(H)
    for b in range(B):
        for h in range(H):
            a1 = softmax_rows(q1[b, h] @ k1[b, h].T * c, vis)
            a2 = softmax_rows(q2[b, h] @ k2[b, h].T * c, vis)
            o1 = a1 @ v[b, h]
            o2 = a2 @ v[b, h]
            o = o1 - lam[h] * o2
            r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
            gy = dy[b, h]
            do = g * r * gy - g * r ** 3 * np.sum(o * gy, axis=-1, keepdims=True) * o / n
            out["dv"][b, h] = a1.T @ do - lam[h] * (a2.T @ do)
            for a, qq, kk, sgn, dq, dk in ((a1, q1, k1, 1.0, "dq1", "dk1"),
                                           (a2, q2, k2, -lam[h], "dq2", "dk2")):
                da = sgn * (do @ v[b, h].T)
                ds = a * (da - np.sum(a * da, axis=-1, keepdims=True))
                out[dq][b, h] = c * (ds @ kk[b, h])
                out[dk][b, h] = c * (ds.T @ qq[b, h])
            dlam[h] += -np.sum(do * o2)
            dlam_terms[h] += np.sum(np.abs(do * o2))
    out["dlam"] = dlam
    # the size of dlambda's terms before they cancel: the scale its rounding error is set by
    out["dlam_terms"] = dlam_terms
    out["dlq1"] = (dlam * ea)[:, None] * lk1
    out["dlk1"] = (dlam * ea)[:, None] * lq1
    out["dlq2"] = -(dlam * eb)[:, None] * lk2
    out["dlk2"] = -(dlam * eb)[:, None] * lq2
    return out

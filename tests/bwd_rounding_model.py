"""A float64 model of where the V1 training forward and backward round to bf16.  TEST SIDE ONLY.

This is not an oracle: it copies the *kernels'* choices (which intermediate is rounded to bf16,
the reference max of the forward's softmax, the log-sum-exp the backward rebuilds its weights
from) so that the backward's tolerance can be derived from the arithmetic rather than picked.
Everything not rounded to bf16 is carried in float64, with float32 rounding only where it feeds
a bf16 decision (exponent arguments and weights), so the model's error against the float64
backward oracle is the error those bf16 roundings alone cause.

What it follows (the V1 layout of Ultralytics glossary "Differential Transformer", section
"Cómo funciona la atención diferencial": two softmax branches over Q_b K_b^T / sqrt(d), their
lambda-weighted difference times V, per-head RMS norm and the (1 - lambda_init) scale):

forward, per branch and 32-row group of query rows (a kernel wavefront):
  * scores s = Q_b K_b^T in float32; keys in tiles of 32;
  * a reference max m per row: the exact max of the row's first tile, moved (with the partial
    sums rescaled) only when some lane's sum of a tile's weights exceeds 2^12 -- a lane holds
    one row and the 16 keys of the tile with (key mod 8) < 4, or the other 16;
  * weights p = exp2(s log2(e)/sqrt(d) - m log2(e)/sqrt(d)) in float32, rounded to bf16 (pr);
  * l = sum of pr, O_b = (sum_j pr_j V_j) / l, and the base-2 log-sum-exp LSE_b = m c + log2(l);
backward:
  * x = O_1 - lambda O_2, dO = g r dy - g r^3 (x . dy) x / 2d rounded to bf16 (g = 1 - lambda_init,
    r = 1 / sqrt(mean(x^2) + eps)), Dt_b = dO . O_b with the rounded dO;
  * P_b = exp2(s c - LSE_b) in float32 (not rounded), X = dO V^T;
  * P' = P_1 - lambda P_2 rounded to bf16 (the dV operand), and dS_b / c_b = P_b (X - Dt_b)
    rounded to bf16 (the dK_b and dQ_b operands), c_1 = 1, c_2 = -lambda;
  * dV = dO^T P', dK_b = c_b dS_b^T Q_b / sqrt(d), dQ_b = c_b dS_b K_b / sqrt(d).

``model_backward`` returns the same dictionary keys as the backward oracle (dq1 ... dv, dlam).
Any flag in ``exact`` switches one rounding point off, which attributes the error to its sources.
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634


def bf16(x):
    """Round float32 values to bf16 (nearest, ties to even); returns float64 values."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _visible(n, causal, window):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= j > i - window
    return vis


def _forward_branch(q, k, v, vis, sl2, round_p=True):
    """One branch of the training forward for one head: returns O_b [n, dv] and LSE_b [n]."""
    n = q.shape[0]
    s = f32(q @ k.T)
    s_m = np.where(vis, s, -np.inf)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    ms = np.zeros(n)
    ls = np.zeros(n)
    lane_hi = ((np.arange(32) >> 2) & 1).astype(bool)  # the lane pair half holding each tile key
    for w0 in range(0, n, 32):
        rows = np.arange(w0, min(n, w0 + 32))
        vis_rows = vis[rows]
        keys_any = np.nonzero(vis_rows.any(axis=0))[0]
        t_first, t_last = keys_any.min() // 32, keys_any.max() // 32
        m = np.full(rows.size, -np.inf)
        acc = np.zeros((rows.size, v.shape[1]))
        l = np.zeros(rows.size)
        for t in range(t_first, t_last + 1):
            ks = slice(32 * t, min(n, 32 * t + 32))
            st = s_m[rows, ks]
            first = t == t_first
            if first:
                m = st.max(axis=1)
                m = np.where(np.isfinite(m), m, -1.0e30)  # a row with no key in this tile yet

            def weights(mm):
                nm = f32(-f32(mm) * sl2)
                e = f32(st * sl2 + nm[:, None])
                with np.errstate(over="ignore"):   # a row whose reference is still -1e30
                    p = f32(np.exp2(e))
                return bf16(p) if round_p else p

            pr = weights(m)
            if not first:
                hi = lane_hi[: pr.shape[1]]
                lane_sums = np.concatenate([pr[:, ~hi].sum(axis=1), pr[:, hi].sum(axis=1)])
                if np.any(~(lane_sums <= 4096.0)):
                    mnew = np.maximum(m, st.max(axis=1))
                    mnew = np.where(np.isfinite(mnew), mnew, -1.0e30)
                    alpha = f32(np.exp2(f32((m - mnew) * sl2)))
                    acc *= alpha[:, None]
                    l *= alpha
                    m = mnew
                    pr = weights(m)
            l += pr.sum(axis=1)
            acc += pr @ v[ks]
        o[rows] = acc / l[:, None]
        lse[rows] = f32(f32(m * sl2) + np.log2(l))
        ms[rows] = m
        ls[rows] = l
    return f32(o), lse, ms, ls


def model_backward(q1, q2, k1, k2, v, lam, lam_init, dy, causal=True, eps=1e-5, window=0,
                   exact=()):
    """Gradients of one V1 layer with the kernels' bf16 rounding points.

    Arrays are float64 [B, H, N, .] holding bf16 (or float32) values; ``lam`` is [H] (the lambda
    the kernels use).  ``exact`` may hold "p_fwd", "do", "pc", "ds" to leave that rounding out.
    """
    B, H, N, d = q1.shape
    sl2 = float(np.float32(LOG2E / math.sqrt(d)))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    g = float(np.float32(1.0 - lam_init))
    vis = _visible(N, causal, window)
    r_do = (lambda x: f32(x)) if "do" in exact else bf16
    r_pc = (lambda x: f32(x)) if "pc" in exact else bf16
    r_ds = (lambda x: f32(x)) if "ds" in exact else bf16
    out = {k: np.zeros_like(a) for k, a in (("dq1", q1), ("dq2", q2), ("dk1", k1), ("dk2", k2),
                                            ("dv", v))}
    out["dlam"] = np.zeros(H)
    for b in range(B):
        for h in range(H):
            lm = float(np.float32(lam[h]))
            o1, lse1, m1, l1 = _forward_branch(q1[b, h], k1[b, h], v[b, h], vis, sl2, "p_fwd" not in exact)
            o2, lse2, m2, l2 = _forward_branch(q2[b, h], k2[b, h], v[b, h], vis, sl2, "p_fwd" not in exact)
            y = dy[b, h]
            x = o1 - lm * o2
            rr = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
            dot = np.sum(x * y, axis=1, keepdims=True)
            dunr = g * rr * y - g * rr ** 3 * dot / x.shape[1] * x
            do = r_do(dunr)
            nd1 = -f32(np.sum(do * o1, axis=1))
            nd2 = -f32(np.sum(do * o2, axis=1))
            out["dlam"][h] += -np.sum(dunr * o2)
            s1 = f32(q1[b, h] @ k1[b, h].T)
            s2 = f32(q2[b, h] @ k2[b, h].T)
            if "consistent" in exact:
                # the backward re-forms the forward's rounded weights against the same reference
                # max and divides by the forward's sum of them
                def rew(s, m, l):
                    nm = f32(-f32(m) * sl2)
                    return bf16(f32(np.exp2(f32(s * sl2 + nm[:, None])))) / l[:, None]
                p1 = np.where(vis, rew(s1, m1, l1), 0.0)
                p2 = np.where(vis, rew(s2, m2, l2), 0.0)
            else:
                p1 = np.where(vis, f32(np.exp2(f32(s1 * sl2 - lse1[:, None]))), 0.0)
                p2 = np.where(vis, f32(np.exp2(f32(s2 * sl2 - lse2[:, None]))), 0.0)
            xx = f32(do @ v[b, h].T)
            pc = r_pc(p1 - lm * p2)
            ds1 = r_ds(p1 * f32(xx + nd1[:, None]))
            ds2 = r_ds(p2 * f32(xx + nd2[:, None]))
            out["dv"][b, h] = pc.T @ do
            out["dk1"][b, h] = scale * (ds1.T @ q1[b, h])
            out["dk2"][b, h] = -lm * scale * (ds2.T @ q2[b, h])
            out["dq1"][b, h] = scale * (ds1 @ k1[b, h])
            out["dq2"][b, h] = -lm * scale * (ds2 @ k2[b, h])
    return out

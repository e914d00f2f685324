"""Independent brute-force version of differential attention in pure Python (lists, math.exp).

TEST INFRASTRUCTURE ONLY.  It follows the step-by-step description in [L] -- ai-engineering.academy,
Phase 10 Lesson 16 "Atención Diferencial (V2)", section "Implementación" (step 1: softmax with
the row maximum subtracted; step 3: one softmax per branch, element-wise difference of the two
weight rows, then the weighted sum of the value rows) -- written independently of
``diffattn_oracle`` (no numpy, no shared helpers).  Meant for tiny inputs (n <= 16) only; the
tests require it to agree with the numpy oracle to ~1e-12.
"""

from __future__ import annotations

import math


def softmax(row):
    """Softmax of a list of floats through its log-normaliser.

    log Z = top + log(sum_j exp(x_j - top)) with top the largest entry (shifting by it keeps every
    exponential at most 1, the stability step of [L] "Implementación", step 1); each weight is then
    exp(x_i - log Z).  ``math.fsum`` keeps the sum exactly rounded.
    """
    top = max(row)
    log_z = top + math.log(math.fsum(math.exp(x - top) for x in row))
    return [math.exp(x - log_z) for x in row]


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def _weights(q, keys, i, causal, scale, window=0):
    """Softmax weights of query row i over the keys it may see, zeros elsewhere.  With a window
    W > 0 (causal only) row i sees keys i - W + 1 .. i."""
    last = i if causal else len(keys) - 1
    first = max(0, i - window + 1) if window else 0
    w = softmax([dot(q, keys[j]) / scale for j in range(first, last + 1)])
    return [0.0] * first + w + [0.0] * (len(keys) - 1 - last)


def diff_attention(Q1, K1, Q2, K2, V, lam, causal=False, window=0):
    """(A1 - lam * A2) V for one head; all arguments are lists of lists of floats."""
    scale = math.sqrt(len(Q1[0]))
    d_v = len(V[0])
    out = []
    for i in range(len(Q1)):
        a1 = _weights(Q1[i], K1, i, causal, scale, window)
        a2 = _weights(Q2[i], K2, i, causal, scale, window)
        w = [x - lam * y for x, y in zip(a1, a2)]
        out.append([sum(wj * V[j][c] for j, wj in enumerate(w)) for c in range(d_v)])
    return out


def attention(Q, K, V, causal=False, window=0):
    """Plain softmax attention softmax(Q K^T / sqrt(d)) V for one head."""
    scale = math.sqrt(len(Q[0]))
    d_v = len(V[0])
    out = []
    for i in range(len(Q)):
        w = _weights(Q[i], K, i, causal, scale, window)
        out.append([sum(wj * V[j][c] for j, wj in enumerate(w)) for c in range(d_v)])
    return out


def rms_normalise(row, eps):
    ms = sum(x * x for x in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [x * r for x in row]


def layer_lambda_init(layer):
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def head_lambda(lq1, lk1, lq2, lk2, layer):
    return math.exp(dot(lq1, lk1)) - math.exp(dot(lq2, lk2)) + layer_lambda_init(layer)


def v1_head(Q1, K1, Q2, K2, V, lam, lam_init, causal, eps):
    """V1 head output: RMS-normalised core rows scaled by (1 - lam_init)."""
    core = diff_attention(Q1, K1, Q2, K2, V, lam, causal)
    return [[x * (1.0 - lam_init) for x in rms_normalise(r, eps)] for r in core]


def v2_pair(Qa, Qb, K, V, lam, causal):
    """V2 pair output: attention of head a minus lam times attention of head b (shared K, V)."""
    oa = attention(Qa, K, V, causal)
    ob = attention(Qb, K, V, causal)
    return [[x - lam * y for x, y in zip(ra, rb)] for ra, rb in zip(oa, ob)]

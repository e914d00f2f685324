"""Plain, slow, float64 CPU oracle of the differential-attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``smoke()`` and the ``cpu_baseline`` leg of
``bench.py``; never by the product path.  It shares no code with the HIP library.

It computes the method's plain definition directly -- two ordinary softmax maps, their
lambda-weighted difference, the product with V, then (V1) a per-head RMS normalisation and the
(1 - lambda_init) scale -- in numpy float64 on the exact input values.  There is no online
softmax, no tiling of the key axis and no fusion: query rows are processed in blocks only to
bound memory, which does not change any arithmetic (rows are independent).  The matmul is the
only library primitive used.

Sources (web pages; cited by title and section):
  [G]  Ultralytics glossary entry "Differential Transformer" (Spanish edition; the Turkish
       edition is a sentence-for-sentence twin), section "Cómo funciona la atención diferencial".
  [L]  ai-engineering.academy, Phase 10 Lesson 16 "Atención Diferencial (V2)", sections
       "El piso de ruido de softmax", "La idea diferencial", "V1 vs V2: la diferencia",
       "Implementación" (steps 1-3) and "Ejercicios" (exercises 4 and 5).

Readings taken where the pages are silent or ambiguous (each is listed in the design doc too):
  * d inside sqrt(d) is the per-branch query/key width ([G] example divides by the half width).
  * causal: key j is visible to query i iff j <= i (square, N_q == N_k); masked weights are 0.
  * sliding window W (the window layers of the hybrid DIFF / sliding-window stacks that [L]
    "Úselo" mentions): causal, and key j is visible to query i only if i - W < j, so each row
    sees its last W positions including itself.  W = 0 means no window.
  * one lambda per head (V1) or per head pair (V2), from rows of four [H, d] vectors.
  * lambda_init uses the 1-based layer index; the V1 norm is RMS (no mean subtraction, no gain),
    eps inside the square root, applied before the (1 - lambda_init) scale; V2 has neither.
  * V2 pairs query heads (2p, 2p+1) over KV head p * Hkv // P and subtracts the pair's outputs.
  * decode: the single new query sits at cache row L-1 and sees all L rows.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lambda_init",
    "lambda_value",
    "softmax_rows",
    "diff_maps",
    "diff_core_rows",
    "branch_rows",
    "rms_norm_rows",
    "diff_attn_v1",
    "diff_attn_v1_layers",
    "diff_attn_v2",
    "diff_decode_v2",
    "diff_decode_v1",
]

# Largest number of score entries (rows x keys) materialised at once per branch.
_MAX_BLOCK_ENTRIES = 1 << 23


def lambda_init(layer: int) -> float:
    """Initial lambda for 1-based layer ``layer``: 0.8 - 0.6 * exp(-0.3 * (layer - 1)).

    [G] "Cómo funciona la atención diferencial": lambda starts from this schedule, so deeper
    layers start nearer 0.8 (layer 1 starts at 0.2).
    """
    layer = int(layer)
    if layer < 1:
        raise ValueError(f"layer index is 1-based, got {layer}")
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def lambda_value(lq1, lk1, lq2, lk2, layer: int) -> np.ndarray:
    """Per-head lambda = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lambda_init(layer).

    [L] "La idea diferencial": lambda is a learnable scalar per head built from four vectors; it
    may be negative and is not clamped.  [G] names the four small vectors and the schedule.
    Arguments are arrays of shape [H, d] (or [d] for a single head); returns float64 [H].
    """
    lq1, lk1, lq2, lk2 = (np.asarray(a, dtype=np.float64) for a in (lq1, lk1, lq2, lk2))
    dot1 = np.sum(lq1 * lk1, axis=-1)
    dot2 = np.sum(lq2 * lk2, axis=-1)
    return np.exp(dot1) - np.exp(dot2) + lambda_init(layer)


def softmax_rows(scores: np.ndarray, visible: np.ndarray | None = None) -> np.ndarray:
    """Exact two-pass softmax along the last axis, subtracting the row maximum first.

    [L] "Implementación", step 1 (max subtraction for numerical stability) and
    "El piso de ruido de softmax" (w_i = exp(s_i) / sum_j exp(s_j)).  Entries with
    ``visible == False`` get weight exactly 0 and do not enter the max or the sum.
    Every row must have at least one visible entry.
    """
    s = np.asarray(scores, dtype=np.float64)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("softmax row with no visible entry")
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _visible(rows: np.ndarray, n_keys: int, causal: bool, window: int = 0) -> np.ndarray | None:
    if window and not causal:
        raise ValueError("a sliding window is defined for causal attention only")
    if not causal:
        return None
    keys = np.arange(n_keys)
    vis = keys[None, :] <= rows[:, None]
    if window:
        vis &= keys[None, :] > rows[:, None] - window
    return vis


def diff_maps(q1, k1, q2, k2, lam: float, causal: bool = False, window: int = 0):
    """Both softmax maps of one head and their lambda-weighted difference.

    A1 = softmax(Q1 K1^T / sqrt(d)), A2 = softmax(Q2 K2^T / sqrt(d)), W = A1 - lam * A2,
    with d the per-branch width ([L] "La idea diferencial"; [G] "Cómo funciona la atención
    diferencial", whose worked example also divides by the square root of the half width).
    Inputs are 2-D [n, d]; returns (A1, A2, W), each [n_q, n_k].
    """
    q1, k1, q2, k2 = (np.asarray(a, dtype=np.float64) for a in (q1, k1, q2, k2))
    d = q1.shape[-1]
    rows = np.arange(q1.shape[0])
    vis = _visible(rows, k1.shape[0], causal, window)
    a1 = softmax_rows(q1 @ k1.T / math.sqrt(d), vis)
    a2 = softmax_rows(q2 @ k2.T / math.sqrt(d), vis)
    return a1, a2, a1 - lam * a2


def _row_blocks(rows: np.ndarray, n_keys: int):
    step = max(1, _MAX_BLOCK_ENTRIES // max(1, n_keys))
    for s in range(0, len(rows), step):
        yield rows[s : s + step]


def _rows_arg(rows, n: int) -> np.ndarray:
    if rows is None:
        return np.arange(n)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= n):
        raise IndexError("query row out of range")
    return rows


def diff_core_rows(q1, k1, q2, k2, v, lam: float, causal: bool, rows=None, window: int = 0) -> np.ndarray:
    """Un-normalised differential attention (A1 - lam * A2) V for chosen query rows of one head.

    [L] "La idea diferencial" (DiffAttn = (A_1 - lambda A_2) V) and "Implementación" step 3;
    [G] "Cómo funciona la atención diferencial" (V twice as wide as each query/key half).
    q*, k* are [n, d], v is [n, dv]; ``rows`` selects query rows (default: all).
    Under ``causal`` only keys j <= i are visible, so the key axis is cut at the last row of
    each block before the products (this changes no value: the cut keys carry weight 0).
    """
    q1, k1, q2, k2, v = (np.asarray(a, dtype=np.float64) for a in (q1, k1, q2, k2, v))
    n_k = k1.shape[0]
    d = q1.shape[-1]
    rows = _rows_arg(rows, q1.shape[0])
    out = np.empty((rows.size, v.shape[-1]), dtype=np.float64)
    pos = 0
    for blk in _row_blocks(rows, n_k):
        kmax = int(blk.max()) + 1 if causal else n_k
        vis = _visible(blk, kmax, causal, window)
        a1 = softmax_rows(q1[blk] @ k1[:kmax].T / math.sqrt(d), vis)
        a2 = softmax_rows(q2[blk] @ k2[:kmax].T / math.sqrt(d), vis)
        out[pos : pos + blk.size] = (a1 - lam * a2) @ v[:kmax]
        pos += blk.size
    return out


def branch_rows(q, k, v, causal: bool, rows=None, window: int = 0) -> np.ndarray:
    """One ordinary softmax-attention branch softmax(q k^T / sqrt(d)) v for chosen query rows.

    Used by the V2 layout, where every query head of a pair runs plain softmax attention
    ([L] "V1 vs V2: la diferencia").  q is [n, D], k and v are [n_k, D].
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n_k = k.shape[0]
    d = q.shape[-1]
    rows = _rows_arg(rows, q.shape[0])
    out = np.empty((rows.size, v.shape[-1]), dtype=np.float64)
    pos = 0
    for blk in _row_blocks(rows, n_k):
        kmax = int(blk.max()) + 1 if causal else n_k
        vis = _visible(blk, kmax, causal, window)
        a = softmax_rows(q[blk] @ k[:kmax].T / math.sqrt(d), vis)
        out[pos : pos + blk.size] = a @ v[:kmax]
        pos += blk.size
    return out


def rms_norm_rows(o: np.ndarray, eps: float) -> np.ndarray:
    """Per-row RMS normalisation y = o / sqrt(mean(o^2) + eps), no mean subtraction, no gain.

    [G] "Cómo funciona la atención diferencial": each head's output is normalised on its own
    (called GroupNorm there); [L] calls the same step the per-head RMSNorm.
    """
    o = np.asarray(o, dtype=np.float64)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)


def diff_attn_v1(q1, q2, k1, k2, v, lam, lam_init: float, causal: bool = True,
                 eps: float = 1e-5, norm: bool = True, rows=None, heads=None, batches=None,
                 window: int = 0):
    """V1 layout: per head, (A1 - lam_h A2) V, then RMS norm and the (1 - lam_init) scale.

    Shapes: q1, q2, k1, k2 [B, H, N, d]; v [B, H, N, 2d]; lam [H] (one lambda per head).
    [G] "Cómo funciona la atención diferencial" (half the heads, V twice as wide, per-head
    normalisation then scaling by one minus the initial lambda); [L] "V1 vs V2: la diferencia".
    ``norm=False`` returns the core (A1 - lam A2) V without normalisation or scale.
    ``rows``/``heads``/``batches`` restrict the evaluation (default: all).  ``window`` > 0
    restricts each row to its last ``window`` positions (causal sliding window).
    Returns float64 [len(batches), len(heads), len(rows), 2d].
    """
    b_list = range(q1.shape[0]) if batches is None else list(batches)
    h_list = range(q1.shape[1]) if heads is None else list(heads)
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), (q1.shape[1],))
    rows = _rows_arg(rows, q1.shape[2])
    out = np.empty((len(b_list), len(h_list), rows.size, v.shape[-1]), dtype=np.float64)
    for bi, b in enumerate(b_list):
        for hi, h in enumerate(h_list):
            o = diff_core_rows(q1[b, h], k1[b, h], q2[b, h], k2[b, h], v[b, h],
                               float(lam[h]), causal, rows, window)
            if norm:
                o = rms_norm_rows(o, eps) * (1.0 - lam_init)
            out[bi, hi] = o
    return out


def diff_attn_v1_layers(q1, q2, k1, k2, v, lams, lam_inits, causal: bool = True,
                        eps: float = 1e-5, rows=None, heads=None, batches=None, window: int = 0):
    """V1 outputs of several layers that share Q1, Q2, K1, K2, V and differ only in lambda.

    (A1 - lam A2) V = A1 V - lam (A2 V) by distributivity, so the two branch outputs A1 V and
    A2 V are formed once per head and each layer's difference, RMS norm and (1 - lambda_init)
    scale is applied to them ([L] "V1 vs V2: la diferencia" states the same identity: the V2
    layout subtracts two heads' ordinary attention outputs and the math is unchanged).
    ``lams`` is [n_layers, H] (one lambda per head and layer), ``lam_inits`` is [n_layers].
    Returns float64 [n_layers, len(batches), len(heads), len(rows), 2d].
    """
    lams = np.asarray(lams, dtype=np.float64)
    lam_inits = np.asarray(lam_inits, dtype=np.float64).reshape(-1)
    if lams.ndim != 2 or lams.shape != (lam_inits.size, q1.shape[1]):
        raise ValueError("lams must be [n_layers, H] with one lambda_init per layer")
    b_list = range(q1.shape[0]) if batches is None else list(batches)
    h_list = range(q1.shape[1]) if heads is None else list(heads)
    rows = _rows_arg(rows, q1.shape[2])
    out = np.empty((lam_inits.size, len(b_list), len(h_list), rows.size, v.shape[-1]),
                   dtype=np.float64)
    for bi, b in enumerate(b_list):
        for hi, h in enumerate(h_list):
            o1 = branch_rows(q1[b, h], k1[b, h], v[b, h], causal, rows, window)
            o2 = branch_rows(q2[b, h], k2[b, h], v[b, h], causal, rows, window)
            for li in range(lam_inits.size):
                out[li, bi, hi] = rms_norm_rows(o1 - lams[li, h] * o2, eps) * (1.0 - lam_inits[li])
    return out


def diff_attn_v2(q, k, v, lam, causal: bool = True, rows=None, pairs=None, batches=None,
                 window: int = 0):
    """V2 layout: query heads doubled and paired over shared KV heads, pair outputs subtracted.

    q [B, 2P, N, D]; k, v [B, Hkv, N, D]; lam [P].  Pair p uses query heads 2p and 2p+1, both
    reading KV head g = p * Hkv // P, and returns O_2p - lam_p * O_2p+1 with no normalisation
    and no scale ([L] "V1 vs V2: la diferencia": doubled query heads, unchanged KV heads,
    outputs subtracted, per-head RMSNorm removed; "Ejercicios" 5: GQA with 32 Q / 8 KV heads).
    Returns float64 [len(batches), len(pairs), len(rows), D].
    """
    n_pairs = q.shape[1] // 2
    hkv = k.shape[1]
    if q.shape[1] != 2 * n_pairs or n_pairs % hkv != 0:
        raise ValueError("need 2P query heads with P a multiple of the KV head count")
    b_list = range(q.shape[0]) if batches is None else list(batches)
    p_list = range(n_pairs) if pairs is None else list(pairs)
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), (n_pairs,))
    rows = _rows_arg(rows, q.shape[2])
    out = np.empty((len(b_list), len(p_list), rows.size, v.shape[-1]), dtype=np.float64)
    for bi, b in enumerate(b_list):
        for pi, p in enumerate(p_list):
            g = p * hkv // n_pairs
            oa = branch_rows(q[b, 2 * p], k[b, g], v[b, g], causal, rows, window)
            ob = branch_rows(q[b, 2 * p + 1], k[b, g], v[b, g], causal, rows, window)
            out[bi, pi] = oa - float(lam[p]) * ob
    return out


def diff_decode_v2(q, kcache, vcache, lam, batches=None, pairs=None):
    """One V2 decode step: each sequence's single new query attends to all L cache rows.

    q [B, 2P, D]; kcache, vcache [B, Hkv, L, D] (row L-1 holds the new token's own K/V);
    lam [P].  The result equals the last row of the V2 prefill at N = L ([L] "V1 vs V2: la
    diferencia": V2 decode reads the KV cache once for both heads of a pair).
    Returns float64 [len(batches), len(pairs), D].
    """
    n_pairs = q.shape[1] // 2
    hkv = kcache.shape[1]
    b_list = range(q.shape[0]) if batches is None else list(batches)
    p_list = range(n_pairs) if pairs is None else list(pairs)
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), (n_pairs,))
    out = np.empty((len(b_list), len(p_list), vcache.shape[-1]), dtype=np.float64)
    for bi, b in enumerate(b_list):
        for pi, p in enumerate(p_list):
            g = p * hkv // n_pairs
            oa = branch_rows(np.asarray(q[b, 2 * p])[None, :], kcache[b, g], vcache[b, g], False)
            ob = branch_rows(np.asarray(q[b, 2 * p + 1])[None, :], kcache[b, g], vcache[b, g], False)
            out[bi, pi] = (oa - float(lam[p]) * ob)[0]
    return out


def diff_decode_v1(q1, q2, k1cache, k2cache, vcache, lam, lam_init: float, eps: float = 1e-5,
                   norm: bool = True):
    """One V1 decode step: the new query of each head attends to all L cache rows.

    q1, q2 [B, H, d]; k1cache, k2cache [B, H, L, d]; vcache [B, H, L, 2d]; lam [H].
    Equals the last row of the V1 prefill at N = L ([L] "V1 vs V2: la diferencia": V1 decode
    needs the value cache for both softmax branches).  Returns float64 [B, H, 2d].
    """
    B, H = q1.shape[0], q1.shape[1]
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), (H,))
    out = np.empty((B, H, vcache.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o = diff_core_rows(np.asarray(q1[b, h])[None, :], k1cache[b, h],
                               np.asarray(q2[b, h])[None, :], k2cache[b, h], vcache[b, h],
                               float(lam[h]), False)
            if norm:
                o = rms_norm_rows(o, eps) * (1.0 - lam_init)
            out[b, h] = o[0]
    return out

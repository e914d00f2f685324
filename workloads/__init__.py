"""Seeded synthetic workloads for the differential-attention forward pass.

This module holds input shapes and seeded random draws only -- none of the method's arithmetic.
Both sides of every parity check (the HIP library through its binding, and the CPU oracle)
receive the same arrays from here, and nothing here imports either side.

Draws
-----
Every tensor is filled chunk by chunk, one chunk per (batch, head) slice, each chunk from its own
PCG64 stream seeded with ``SeedSequence([seed, tensor_tag, b, h])``.  The values therefore do not
depend on the number of threads used to fill them.  Activations are i.i.d. N(0, 1); the four
lambda vectors are i.i.d. N(0, 0.1^2).  bf16 inputs are fp32 draws rounded to bf16 with
round-to-nearest-even; the oracle reads exactly those bf16 values.

Workloads
---------
``CONFIGS`` lists the workloads: a small fp32 V1 case, the V1 prefill at a 4K context, the V2
(GQA, paired query heads) prefill at 8K, the V2 decode step over a 32K-token cache, the V1
long-context prefill at 128K tokens with planted "needle" keys, the V1-layout decode step
over a 32K-token cache (its K1 + K2 + V cache is as large as the V2 decode's K + V cache), and
the V1 prefill at 4K restricted to a causal sliding window of 1024 keys, and the V2 decode step
on a paged KV cache (16-key pages in a random order, per-sequence lengths 4K .. 32K).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ---------------------------------------------------------------------------------------------
# workload table
# ---------------------------------------------------------------------------------------------

CONFIGS = {
    "v1_fp32_small": dict(kind="v1", dtype="f32", B=1, H=2, N=128, d=64, causal=True,
                          layers=(1, 2, 3, 4), eps=1e-5, seed=1001),
    "v1_prefill_4k": dict(kind="v1", dtype="bf16", B=4, H=16, N=4096, d=64, causal=True,
                          layers=(12,), eps=1e-5, seed=1002),
    "v2_prefill_8k": dict(kind="v2", dtype="bf16", B=2, P=16, Hkv=8, N=8192, D=128, causal=True,
                          layers=(24,), seed=1003),
    "v2_decode_32k": dict(kind="decode", dtype="bf16", B=64, P=16, Hkv=8, L=32768, D=128,
                          layers=(24,), seed=1004),
    "v1_long_128k": dict(kind="v1", dtype="bf16", B=1, H=16, N=131072, d=64, causal=True,
                         layers=tuple(range(1, 33)), eps=1e-5, needles=6, seed=1005),
    "v1_decode_32k": dict(kind="decode_v1", dtype="bf16", B=32, H=16, L=32768, d=64,
                          layers=(12,), eps=1e-5, seed=1006),
    "v1_swa_4k": dict(kind="v1", dtype="bf16", B=4, H=16, N=4096, d=64, causal=True, window=1024,
                      layers=(12,), eps=1e-5, seed=1007),
    "v2_decode_paged": dict(kind="decode_paged", dtype="bf16", B=64, P=16, Hkv=8, D=128,
                            page_size=16, len_lo=4096, len_hi=32768, layers=(24,), seed=1008),
}

_TAGS = {"q1": 1, "q2": 2, "k1": 3, "k2": 4, "v": 5, "q": 6, "k": 7,
         "lq1": 11, "lk1": 12, "lq2": 13, "lk2": 14, "needle": 21}

LAMBDA_STD = 0.1


def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(16, n))


# ---------------------------------------------------------------------------------------------
# bf16 encoding (input preparation only)
# ---------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite normal draws, so no NaN/Inf special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# seeded fills
# ---------------------------------------------------------------------------------------------

def _stream(seed: int, tag: str, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag], *idx])))


def normal_tensor(seed: int, tag: str, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    """Seeded N(0, std^2) tensor of shape [B, H, ...].

    dtype "f32" returns float32 values; dtype "bf16" returns uint16 bf16 bit patterns.
    """
    shape = tuple(int(s) for s in shape)
    B, H = shape[0], shape[1]
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        x = _stream(seed, tag, b, h).standard_normal(shape[2:], dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[b, h] = x if dtype == "f32" else f32_to_bf16_bits(x)

    n = B * H
    if n * int(np.prod(shape[2:], dtype=np.int64)) < (1 << 22):
        for bh in range(n):
            fill(bh)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n)))
    return out


def lambda_vectors(seed: int, n: int, dl: int, layer: int):
    """The four lambda vectors (lq1, lk1, lq2, lk2), float32 [n, dl] each, N(0, 0.1^2), per layer."""
    return tuple(
        (_stream(seed, t, layer, 0).standard_normal((n, dl), dtype=np.float32)
         * np.float32(LAMBDA_STD)).astype(np.float32)
        for t in ("lq1", "lk1", "lq2", "lk2"))


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values of a generated tensor (identity for f32, exact decode for bf16 bits)."""
    return x if dtype == "f32" else bf16_bits_to_f32(x)


# ---------------------------------------------------------------------------------------------
# whole workloads
# ---------------------------------------------------------------------------------------------

def make_v1(B, H, N, d, dtype="bf16", seed=0, needles=0, layers=(1,)):
    """V1 inputs: q1, q2, k1, k2 [B, H, N, d]; v [B, H, N, 2d]; lambda vectors [H, d] per layer.

    With ``needles`` > 0, for every (b, h) the last query row i* = N-1 picks that many distinct
    key positions j < i* (seeded) and sets K1[j] to 4 times the unit vector along Q1[i*]
    (rounded to the tensor's dtype).  Only branch 1 gets the needles.
    """
    t = {
        "q1": normal_tensor(seed, "q1", (B, H, N, d), dtype),
        "q2": normal_tensor(seed, "q2", (B, H, N, d), dtype),
        "k1": normal_tensor(seed, "k1", (B, H, N, d), dtype),
        "k2": normal_tensor(seed, "k2", (B, H, N, d), dtype),
        "v": normal_tensor(seed, "v", (B, H, N, 2 * d), dtype),
    }
    t["needle_pos"] = None
    if needles:
        if N < needles + 1:
            raise ValueError("sequence too short for the requested needles")
        pos = np.empty((B, H, needles), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                rng = _stream(seed, "needle", b, h)
                pos[b, h] = np.sort(rng.choice(N - 1, size=needles, replace=False))
                qdir = as_f32(t["q1"][b, h, N - 1], dtype).astype(np.float64)
                key = (4.0 * qdir / np.linalg.norm(qdir)).astype(np.float32)
                enc = key if dtype == "f32" else f32_to_bf16_bits(key)
                t["k1"][b, h, pos[b, h]] = enc
        t["needle_pos"] = pos
    t["lambda"] = {l: lambda_vectors(seed, H, d, l) for l in layers}
    return t


def make_v2(B, P, Hkv, N, D, dtype="bf16", seed=0, layers=(1,)):
    """V2 inputs: q [B, 2P, N, D] (pair p = heads 2p, 2p+1); k, v [B, Hkv, N, D]; lambda [P, D]."""
    return {
        "q": normal_tensor(seed, "q", (B, 2 * P, N, D), dtype),
        "k": normal_tensor(seed, "k", (B, Hkv, N, D), dtype),
        "v": normal_tensor(seed, "v", (B, Hkv, N, D), dtype),
        "lambda": {l: lambda_vectors(seed, P, D, l) for l in layers},
    }


def make_decode(B, P, Hkv, L, D, dtype="bf16", seed=0, layers=(1,)):
    """V2 decode inputs: q [B, 2P, D] (one new token per sequence); kcache, vcache [B, Hkv, L, D]."""
    q = normal_tensor(seed, "q", (B, 2 * P, 1, D), dtype)[:, :, 0, :].copy()
    return {
        "q": q,
        "kcache": normal_tensor(seed, "k", (B, Hkv, L, D), dtype),
        "vcache": normal_tensor(seed, "v", (B, Hkv, L, D), dtype),
        "lambda": {l: lambda_vectors(seed, P, D, l) for l in layers},
    }


def make_decode_v1(B, H, L, d, dtype="bf16", seed=0, layers=(1,)):
    """V1 decode inputs: q1, q2 [B, H, d] (one new token per sequence); k1cache, k2cache
    [B, H, L, d]; vcache [B, H, L, 2d]."""
    return {
        "q1": normal_tensor(seed, "q1", (B, H, 1, d), dtype)[:, :, 0, :].copy(),
        "q2": normal_tensor(seed, "q2", (B, H, 1, d), dtype)[:, :, 0, :].copy(),
        "k1cache": normal_tensor(seed, "k1", (B, H, L, d), dtype),
        "k2cache": normal_tensor(seed, "k2", (B, H, L, d), dtype),
        "vcache": normal_tensor(seed, "v", (B, H, L, 2 * d), dtype),
        "lambda": {l: lambda_vectors(seed, H, d, l) for l in layers},
    }


def make_decode_paged(B, P, Hkv, D, page_size, seq_lens, dtype="bf16", seed=0, layers=(1,)):
    """V2 decode inputs in the serving layout: q [B, 2P, D]; a pool of KV pages
    [num_pages, Hkv, page_size, D]; block_table [B, max_blocks] (pages dealt in a seeded random
    order, unused entries -1); seq_lens [B].  Every page of the pool is drawn N(0, 1)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    blocks = [(int(n) + page_size - 1) // page_size for n in seq_lens]
    num_pages = int(sum(blocks))
    max_blocks = max(blocks)
    order = _stream(seed, "needle", 0, 0).permutation(num_pages).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, nb in enumerate(blocks):
        table[b, :nb] = order[pos:pos + nb]
        pos += nb
    q = normal_tensor(seed, "q", (B, 2 * P, 1, D), dtype)[:, :, 0, :].copy()
    return {
        "q": q,
        "k_pages": normal_tensor(seed, "k", (num_pages, Hkv, page_size, D), dtype),
        "v_pages": normal_tensor(seed, "v", (num_pages, Hkv, page_size, D), dtype),
        "block_table": table,
        "seq_lens": seq_lens,
        "lambda": {l: lambda_vectors(seed, P, D, l) for l in layers},
    }


def paged_lens(B, lo, hi, seed):
    """Seeded per-sequence lengths, uniform in [lo, hi]."""
    return _stream(seed, "needle", 1, 0).integers(lo, hi + 1, size=B).astype(np.int32)


def make(name: str, **overrides):
    """Inputs of a named workload (``CONFIGS``), with optional shape overrides."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg["kind"]
    if kind == "v1":
        return cfg, make_v1(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["dtype"], cfg["seed"],
                            cfg.get("needles", 0), cfg["layers"])
    if kind == "v2":
        return cfg, make_v2(cfg["B"], cfg["P"], cfg["Hkv"], cfg["N"], cfg["D"], cfg["dtype"],
                            cfg["seed"], cfg["layers"])
    if kind == "decode":
        return cfg, make_decode(cfg["B"], cfg["P"], cfg["Hkv"], cfg["L"], cfg["D"], cfg["dtype"],
                                cfg["seed"], cfg["layers"])
    if kind == "decode_paged":
        lens = paged_lens(cfg["B"], cfg["len_lo"], cfg["len_hi"], cfg["seed"])
        return cfg, make_decode_paged(cfg["B"], cfg["P"], cfg["Hkv"], cfg["D"], cfg["page_size"], lens,
                                      cfg["dtype"], cfg["seed"], cfg["layers"])
    if kind == "decode_v1":
        return cfg, make_decode_v1(cfg["B"], cfg["H"], cfg["L"], cfg["d"], cfg["dtype"], cfg["seed"],
                                   cfg["layers"])
    raise KeyError(kind)

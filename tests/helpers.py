"""Shared helpers of the GPU tests: moving seeded numpy inputs to the device and running the
library and the oracle on the same values."""

from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads as wl


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype="bf16"):
    import torch

    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(x).to("cuda")


def dev_lambda(vecs):
    import torch

    return [torch.from_numpy(np.ascontiguousarray(v)).to("cuda") for v in vecs]


def f64(x, dtype="bf16"):
    return wl.as_f32(x, dtype).astype(np.float64)


def oracle_lambda(vecs, layer):
    return oracle.lambda_value(*vecs, layer)


def sample_rows(n, k, seed, extra=()):
    """k distinct rows of [0, n) (seeded) plus the listed extra rows, sorted."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    rows.update(r for r in extra if 0 <= r < n)
    return np.array(sorted(rows), dtype=np.int64)


def parallel_map(fn, items, threads=None):
    """fn over items on a thread pool (numpy releases the GIL in its kernels), with BLAS held to
    one thread per worker so the workers do not oversubscribe the host cores."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    n = threads or max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(1):
        with ThreadPoolExecutor(n) as ex:
            return list(ex.map(fn, items))


def merge_stats(stats):
    """One bf16 verdict over several compared pieces of an output: the max error over all of them
    and the share of within-bound elements over all their elements together (the bar applies to
    the output tensor; a piece of a few thousand elements is too small a sample for 99.9 %)."""
    n = sum(s["n"] for s in stats)
    within = sum(s["frac_within"] * s["n"] for s in stats)
    return {"max_abs": max(s["max_abs"] for s in stats), "frac_within": within / max(n, 1), "n": n,
            "finite": all(s["finite"] for s in stats)}


def bf16_ulps(got, ref):
    """Distance in bf16 steps between bf16 values `got` and the exact `ref` rounded to bf16
    (nearest, ties to even): 0 where the result is the correctly rounded value."""
    import workloads as wl

    def ordered(bits):
        bits = bits.astype(np.int64)
        return np.where(bits & 0x8000, -(bits & 0x7FFF), bits & 0x7FFF)

    g = (np.asarray(got, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = wl.f32_to_bf16_bits(np.asarray(ref, dtype=np.float32))
    return np.abs(ordered(g) - ordered(r))

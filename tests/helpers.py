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
    """One bf16 decision over several compared pieces of an output: the max error over all of them
    and the share of within-bound elements over all their elements together (the bar applies to
    the output tensor; a piece of a few thousand elements is too small a sample for 99.9 %)."""
    n = sum(s["n"] for s in stats)
    within = sum(s["frac_within"] * s["n"] for s in stats)
    return {"max_abs": max(s["max_abs"] for s in stats), "frac_within": within / max(n, 1), "n": n,
            "finite": all(s["finite"] for s in stats)}


def beyond_output_rounding(got, ref):
    """Largest error of `got` beyond what rounding the exact `ref` to bf16 can cause, relative to
    the RMS of each reference row: max of (|got - ref| - 2^-8 |ref|) / rms(ref row), where 2^-8
    |x| bounds half a bf16 step at x.  A path whose only error is the final bf16 store gives
    (nearly) zero here; the remainder is its arithmetic before the store."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    rms = np.where(rms > 0, rms, 1.0)
    return float(np.max((np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)) / rms))

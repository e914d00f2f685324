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

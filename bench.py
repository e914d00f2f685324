"""Benchmark of the differential-attention hot path on one MI355X.

A step is one pass of the hot path over one batch of seeded synthetic input already resident in
HBM.  The headline workload is the largest single-GPU configuration: the V1 prefill at a
128K-token context (B=1, H=16, N=131072, d=64, V width 128, causal, bf16 in / fp32 accumulate,
6 planted needle keys per head), one launch per step, the launches cycling through the layers
l = 1..32 of the lambda sweep (each with its own lambda vectors and lambda_init).  Its line
carries the MFMA roofline and the CPU oracle baseline (on sampled rows of the same workload).
The same JSON line carries, under "secondary", each with its own roofline: the V1 prefill at a 4K
context (B=4, H=16, N=4096, layer 12, with its own oracle baseline), the V2 prefill (B=2, 32 query
heads / 16 pairs over 8 KV heads, D=128, N=8192), the V2 decode step (B=64, 32 query / 8 KV heads,
D=128, 32K-token cache), the same decode over a paged cache with ragged lengths, the V1 prefill
under a 1024-key sliding window, the V1-layout decode step, the V1 backward at the 4K training
shape, causal and under the same window, and a whole V1 training step of the attention
(training forward + backward).

Timing: each workload first runs for SETTLE_S seconds untimed (the shader clock ramps up over
the first tens of milliseconds of load), then W warm-up steps, then K steps between two HIP events
on the stream the kernels run on.  The shader clock is sampled during the timed steps and
reported (median MHz) where the platform exposes it.

FLOP and byte conventions (per launch):
  V1 prefill  algorithmic flops  = B*H * 8*d * Np      (two QK^T products + one (A1-lambda A2)V)
              executed MFMA flops = B*H * 12*d * Np    (two QK^T + two P.V in one fused pass)
  V2 prefill  algorithmic flops  = B*P * 6*D * Np,  executed = B*P * 8*D * Np  (the time includes
              the pass that rewrites V as fp16 for the P.V products)
  decode      algorithmic bytes  = K and V cache + queries + output (every byte read once)
  V1 backward algorithmic flops  = B*H * 16*d * Np   (dO V^T, dV, and dQ_b, dK_b per branch)
              executed MFMA flops = B*H * 28*d * Np  (scores and dO V^T formed in both kernels)
with Np = N(N+1)/2 causal query-key pairs (the window's visible pairs for the sliding window).
timing.shader_clock_mhz_median is the AMD SMI GFX clock reading sampled during the timed steps:
indicative only (the effective clock, counted cycles over kernel time, is what the rocprofv3
counter summaries give); a timed region too short for 20 readings (timing.shader_clock_samples)
gives null, since a handful of readings can land on idle values.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
       [--only long|v1|v2|decode|decode_v1|swa|paged|bwd|bwd_swa|train]
       [--no-cpu-baseline] [--cpu-seconds S]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "diff-attn fwd TFLOP/s (% bf16 MFMA peak); decode HBM GB/s (% of 8 TB/s)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill": os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc", "prefill_bf16.hip"),
    "prefill_v2": os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc", "prefill_v2_bf16.hip"),
    "decode": os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc", "decode_v2.hip"),
    "decode_v1": os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc", "decode_v1.hip"),
    "bwd": os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc", "bwd_v1.hip"),
}


# Headers shared by every kernel family: launch parameters, the workgroup order (head chunks)
# and the load/store helpers, which change what a kernel reads as much as its own source does.
SHARED_SOURCES = [os.path.join(ROOT, "differential_softmax_attention_diff_amd", "csrc", f)
                  for f in ("params.hpp", "launch.hpp", "device_common.hpp", "tile_common.hpp")]


def compile_flags(kind: str) -> list:
    """The kernel family's compile flags, without the machine-specific include paths."""
    from differential_softmax_attention_diff_amd import _build

    flags, skip = [], False
    for f in [*_build.COMMON_FLAGS, *_build.EXTRA_FLAGS.get(os.path.basename(KERNEL_SOURCES[kind]), [])]:
        if skip or f == "-I":
            skip = f == "-I"
            continue
        flags.append(f)
    return flags


def source_hash(kind: str) -> str:
    """sha256[:16] over the kernel family's source, the shared headers and its compile flags."""
    h = hashlib.sha256()
    for path in [KERNEL_SOURCES[kind], *SHARED_SOURCES]:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(compile_flags(kind)).encode())
    return h.hexdigest()[:16]


def combined_hash(kinds) -> str:
    """source_hash of one kernel family, or sha256[:16] over those of several (in order)."""
    if isinstance(kinds, str):
        return source_hash(kinds)
    return hashlib.sha256("+".join(source_hash(k) for k in kinds).encode()).hexdigest()[:16]


def measured_traffic(key: str, kinds):
    """HBM bytes per launch (or step) from the committed counter run, or None if any of the
    kernel families it covers has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("source_hash") != combined_hash(kinds):
        return None
    return ent.get("bytes_per_launch")


def to_dev(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")


SETTLE_S = 0.3   # untimed load before the warm-up steps, so that the shader clock has ramped up


class ClockSampler:
    """Samples the GPU's shader (GFX) clock from a background thread through AMD SMI while the
    timed steps run; ``median_mhz`` is None where the library or the sensor is unavailable, or
    where the timed region was too short for ``MIN_SAMPLES`` readings."""

    def __init__(self, period_s=0.005):
        self.period_s = period_s
        self.samples = []
        self._stop = None
        self._thread = None
        self._smi = None
        self._handle = None

    def __enter__(self):
        import threading

        try:
            import amdsmi

            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._smi, self._handle = amdsmi, handles[0]
        except Exception:  # noqa: BLE001 - no SMI: no clock figure
            self._smi = None
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    info = self._smi.amdsmi_get_clock_info(self._handle, self._smi.AmdSmiClkType.GFX)
                    if isinstance(info.get("clk"), (int, float)):
                        self.samples.append(float(info["clk"]))
                except Exception:  # noqa: BLE001
                    pass
                self._stop.wait(self.period_s)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=1.0)
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass
        return False

    MIN_SAMPLES = 20  # a timed region of a few milliseconds gets a handful of readings, some idle

    @property
    def median_mhz(self):
        return float(np.median(self.samples)) if len(self.samples) >= self.MIN_SAMPLES else None


def time_launches(fn, steps, warmup, torch, settle_s=SETTLE_S):
    """Average milliseconds per call over `steps` calls, HIP events on the stream the kernels are
    launched on, after `settle_s` seconds of untimed calls and `warmup` untimed calls.  Returns
    (ms, info) with the settle launches and the sampled shader clock."""
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    settle = 0
    while time.perf_counter() - t0 < settle_s:
        for _ in range(4):
            fn()
        settle += 4
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clk:
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return ms, {"settle_launches": settle, "shader_clock_mhz_median": clk.median_mhz,
                "shader_clock_samples": len(clk.samples)}


def causal_pairs(n):
    return n * (n + 1) // 2


# ------------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------------

def bench_v1(da, torch, steps, warmup):
    cfg, t = wl.make("v1_prefill_4k")
    layer = cfg["layers"][0]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    args = [to_dev(t[k], torch) for k in ("q1", "q2", "k1", "k2", "v")]
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    out = torch.empty((B, H, N, 2 * d), dtype=torch.bfloat16, device="cuda")
    fn = lambda: da.diffattn_fwd_v1(*args, *lv, layer=layer, out=out)
    ms, timing = time_launches(fn, steps, warmup, torch)
    npairs = causal_pairs(N)
    f_alg = B * H * 8 * d * npairs
    f_exec = B * H * 12 * d * npairs
    tf_alg = f_alg / (ms * 1e-3) / 1e12
    tf_exec = f_exec / (ms * 1e-3) / 1e12
    res = {
        "workload": "v1_prefill_4k", "ms": ms, "timing": timing, "tflops_alg": tf_alg, "tflops_exec": tf_exec,
        "config": {"workload": "v1_prefill_4k", "B": B, "H": H, "N": N, "d": d, "dv": 2 * d,
                   "causal": True, "layer": layer, "dtype": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(tf_alg, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_alg / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("v1_prefill_4k", "prefill"),
                     "executed_mfma_tflops": round(tf_exec, 2),
                     "executed_mfma_frac": round(tf_exec / PEAK_BF16_TFLOPS, 4),
                     "kernel": "prefill_kernel<64,2>"},
    }
    return res, (cfg, t)


def bench_v2(da, torch, steps, warmup):
    cfg, t = wl.make("v2_prefill_8k")
    layer = cfg["layers"][0]
    B, P, Hkv, N, D = cfg["B"], cfg["P"], cfg["Hkv"], cfg["N"], cfg["D"]
    q = to_dev(t["q"], torch)
    k, v = to_dev(t["k"], torch), to_dev(t["v"], torch)
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    out = torch.empty((B, P, N, D), dtype=torch.bfloat16, device="cuda")
    q1, q2 = q[:, 0::2], q[:, 1::2]
    ws = torch.empty(da.diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D), dtype=torch.uint8, device="cuda")
    fn = lambda: da.diffattn_fwd_v2(q1, q2, k, v, *lv, layer=layer, out=out, workspace=ws)
    ms, timing = time_launches(fn, steps, warmup, torch)
    npairs = causal_pairs(N)
    f_alg = B * P * 6 * D * npairs
    f_exec = B * P * 8 * D * npairs
    tf_alg = f_alg / (ms * 1e-3) / 1e12
    tf_exec = f_exec / (ms * 1e-3) / 1e12
    return {
        "workload": "v2_prefill_8k", "ms": ms, "timing": timing, "value": round(tf_alg, 2), "unit": "TFLOP/s",
        "config": {"workload": "v2_prefill_8k", "B": B, "P": P, "query_heads": 2 * P, "Hkv": Hkv,
                   "N": N, "D": D, "causal": True, "layer": layer,
                   "dtype": "bf16 in; Q K^T on bf16 MFMA; P.V on fp16 MFMA (P and a per-call fp16 "
                            "copy of V); fp32 accumulate; bf16 out"},
        "roofline": {"bound": "mfma", "achieved": round(tf_alg, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_alg / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("v2_prefill_8k", "prefill_v2"),
                     "executed_mfma_tflops": round(tf_exec, 2),
                     "executed_mfma_frac": round(tf_exec / PEAK_BF16_TFLOPS, 4),
                     "kernel": "v2_values_kernel + prefill_v2_kernel"},
    }


def bench_long(da, torch, steps, warmup):
    """V1 prefill at a 128K-token context with planted needles, one launch per step; launch i uses
    layer 1 + i % 32, so 32 steps sweep the lambda schedule (one layer per launch).  Returns the
    line and the inputs (kept for the CPU baseline)."""
    cfg, t = wl.make("v1_long_128k")
    layers = cfg["layers"]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    args = [to_dev(t[k], torch) for k in ("q1", "q2", "k1", "k2", "v")]
    lvs = [[torch.from_numpy(x).to("cuda") for x in t["lambda"][l]] for l in layers]
    out = torch.empty((B, H, N, 2 * d), dtype=torch.bfloat16, device="cuda")
    count = [0]

    def fn():
        i = count[0] % len(layers)
        count[0] += 1
        da.diffattn_fwd_v1(*args, *lvs[i], layer=layers[i], out=out)

    # about 0.1 s per launch; launch i uses layer 1 + i % 32 (32 timed steps cover the sweep)
    ms, timing = time_launches(fn, steps, warmup, torch)
    npairs = causal_pairs(N)
    f_alg = B * H * 8 * d * npairs
    f_exec = B * H * 12 * d * npairs
    tf_alg = f_alg / (ms * 1e-3) / 1e12
    tf_exec = f_exec / (ms * 1e-3) / 1e12
    return {
        "workload": "v1_long_128k", "ms": ms, "timing": timing, "value": round(tf_alg, 2), "unit": "TFLOP/s",
        "config": {"workload": "v1_long_128k", "B": B, "H": H, "N": N, "d": d, "dv": 2 * d,
                   "causal": True, "layers": f"{layers[0]}..{layers[-1]} (one per launch)",
                   "needles_per_head": cfg["needles"], "dtype": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(tf_alg, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_alg / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("v1_long_128k", "prefill"),
                     "executed_mfma_tflops": round(tf_exec, 2),
                     "executed_mfma_frac": round(tf_exec / PEAK_BF16_TFLOPS, 4),
                     "kernel": "prefill_kernel<64,2>"},
    }, (cfg, t)


def bench_decode(da, torch, steps, warmup):
    cfg, t = wl.make("v2_decode_32k")
    layer = cfg["layers"][0]
    B, P, Hkv, L, D = cfg["B"], cfg["P"], cfg["Hkv"], cfg["L"], cfg["D"]
    q = to_dev(t["q"], torch)
    kc, vc = to_dev(t["kcache"], torch), to_dev(t["vcache"], torch)
    del t["kcache"], t["vcache"]
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    out = torch.empty((B, P, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(da.diffattn_decode_workspace_bytes(B, P, Hkv, L, D), dtype=torch.uint8,
                     device="cuda")
    q1, q2 = q[:, 0::2], q[:, 1::2]
    fn = lambda: da.diffattn_decode(q1, q2, kc, vc, *lv, layer=layer, out=out, workspace=ws)
    ms, timing = time_launches(fn, steps, warmup, torch)
    nbytes = 2 * B * Hkv * L * D * 2 + B * 2 * P * D * 2 + B * P * D * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "v2_decode_32k", "ms": ms, "timing": timing, "value": round(gbs, 1), "unit": "GB/s",
        "config": {"workload": "v2_decode_32k", "B": B, "P": P, "query_heads": 2 * P, "Hkv": Hkv,
                   "L": L, "D": D, "layer": layer, "dtype": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("v2_decode_32k", "decode"),
                     "algorithmic_bytes": nbytes,
                     "kernel": "decode_partial_kernel<4> + decode_combine_kernel (whole step)"},
    }


def window_pairs(n, w):
    """Visible (query, key) pairs of a causal sliding window of w keys over n rows."""
    w = min(w, n)
    return w * (w + 1) // 2 + (n - w) * w


def bench_swa(da, torch, steps, warmup):
    cfg, t = wl.make("v1_swa_4k")
    layer, window = cfg["layers"][0], cfg["window"]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    args = [to_dev(t[k], torch) for k in ("q1", "q2", "k1", "k2", "v")]
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    out = torch.empty((B, H, N, 2 * d), dtype=torch.bfloat16, device="cuda")
    fn = lambda: da.diffattn_fwd_v1(*args, *lv, layer=layer, out=out, window=window)
    ms, timing = time_launches(fn, steps, warmup, torch)
    npairs = window_pairs(N, window)
    tf_alg = B * H * 8 * d * npairs / (ms * 1e-3) / 1e12
    tf_exec = B * H * 12 * d * npairs / (ms * 1e-3) / 1e12
    return {
        "workload": "v1_swa_4k", "ms": ms, "timing": timing, "value": round(tf_alg, 2), "unit": "TFLOP/s",
        "config": {"workload": "v1_swa_4k", "B": B, "H": H, "N": N, "d": d, "dv": 2 * d,
                   "window": window, "layer": layer, "dtype": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(tf_alg, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_alg / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("v1_swa_4k", "prefill"),
                     "executed_mfma_tflops": round(tf_exec, 2),
                     "executed_mfma_frac": round(tf_exec / PEAK_BF16_TFLOPS, 4),
                     "kernel": "prefill_kernel<64,2> (sliding window)"},
    }


def bench_decode_paged(da, torch, steps, warmup):
    cfg, t = wl.make("v2_decode_paged")
    layer = cfg["layers"][0]
    B, P, Hkv, D, ps = cfg["B"], cfg["P"], cfg["Hkv"], cfg["D"], cfg["page_size"]
    q = to_dev(t["q"], torch)
    kp, vp = to_dev(t["k_pages"], torch), to_dev(t["v_pages"], torch)
    del t["k_pages"], t["v_pages"]
    bt = torch.from_numpy(t["block_table"]).to("cuda")
    sl = torch.from_numpy(t["seq_lens"]).to("cuda")
    max_len = int(t["seq_lens"].max())
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    out = torch.empty((B, P, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(da.diffattn_decode_workspace_bytes(B, P, Hkv, max_len, D), dtype=torch.uint8,
                     device="cuda")
    q1, q2 = q[:, 0::2], q[:, 1::2]
    fn = lambda: da.diffattn_decode_paged(q1, q2, kp, vp, bt, sl, *lv, layer=layer, max_len=max_len,
                                          out=out, workspace=ws)
    ms, timing = time_launches(fn, steps, warmup, torch)
    keys = int(t["seq_lens"].sum())
    # every live key's K and V rows once, the block table, q and out
    nbytes = 2 * keys * Hkv * D * 2 + t["block_table"].nbytes + B * 2 * P * D * 2 + B * P * D * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "v2_decode_paged", "ms": ms, "timing": timing, "value": round(gbs, 1), "unit": "GB/s",
        "config": {"workload": "v2_decode_paged", "B": B, "P": P, "query_heads": 2 * P, "Hkv": Hkv,
                   "D": D, "page_size": ps, "seq_len_range": [cfg["len_lo"], cfg["len_hi"]],
                   "total_keys": keys, "layer": layer, "dtype": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("v2_decode_paged", "decode"),
                     "algorithmic_bytes": nbytes,
                     "kernel": "decode_paged_balanced_kernel<4> + decode_combine_kernel (whole step)"},
    }


def bench_decode_v1(da, torch, steps, warmup):
    cfg, t = wl.make("v1_decode_32k")
    layer = cfg["layers"][0]
    B, H, L, d = cfg["B"], cfg["H"], cfg["L"], cfg["d"]
    q1, q2 = to_dev(t["q1"], torch), to_dev(t["q2"], torch)
    k1, k2, vc = (to_dev(t[k], torch) for k in ("k1cache", "k2cache", "vcache"))
    del t["k1cache"], t["k2cache"], t["vcache"]
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    out = torch.empty((B, H, 2 * d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(da.diffattn_decode_v1_workspace_bytes(B, H, L, d), dtype=torch.uint8,
                     device="cuda")
    fn = lambda: da.diffattn_decode_v1(q1, q2, k1, k2, vc, *lv, layer=layer, out=out, workspace=ws)
    ms, timing = time_launches(fn, steps, warmup, torch)
    # K1 + K2 + V read once, the two query halves read, the output written
    nbytes = B * H * L * (d + d + 2 * d) * 2 + 2 * B * H * d * 2 + B * H * 2 * d * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "v1_decode_32k", "ms": ms, "timing": timing, "value": round(gbs, 1), "unit": "GB/s",
        "config": {"workload": "v1_decode_32k", "B": B, "H": H, "L": L, "d": d, "dv": 2 * d,
                   "layer": layer, "dtype": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("v1_decode_32k", "decode_v1"),
                     "algorithmic_bytes": nbytes,
                     "kernel": "decode_v1_partial_kernel + decode_v1_combine_kernel (whole step)"},
    }


def bench_bwd_v1(da, torch, steps, warmup, window=0):
    """V1 backward at the 4K prefill shape (optionally under the 1024-key sliding window of the
    window workload): the training forward fills the stash once, then the backward (prep, dK/dV,
    dQ and lambda kernels) is timed."""
    name = "v1_swa_backward_4k" if window else "v1_backward_4k"
    cfg, t = wl.make("v1_swa_4k" if window else "v1_prefill_4k")
    layer = cfg["layers"][0]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    args = [to_dev(t[k], torch) for k in ("q1", "q2", "k1", "k2", "v")]
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    rng = np.random.default_rng(77)
    dy = to_dev(wl.f32_to_bf16_bits(rng.standard_normal((B, H, N, 2 * d), dtype=np.float32)), torch)
    _, stash = da.diffattn_fwd_v1_train(*args, *lv, layer=layer, window=window)
    ws = torch.empty(da.diffattn_bwd_v1_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    grads = da.diffattn_bwd_v1(*args, dy, *lv, layer=layer, stash=stash, workspace=ws, window=window)
    fn = lambda: da.diffattn_bwd_v1(*args, dy, *lv, layer=layer, stash=stash, workspace=ws,
                                    grads=grads, window=window)
    ms, timing = time_launches(fn, steps, warmup, torch)
    npairs = window_pairs(N, window) if window else causal_pairs(N)
    # gradient products: dP = dO V^T and dV = (A1 - lambda A2)^T dO (2d wide, once each), and
    # dQ_b = dS_b K_b, dK_b = dS_b^T Q_b per branch
    f_alg = B * H * 16 * d * npairs
    # executed: dK/dV kernel S_1, S_2, X = dO V^T, dV, dK_1, dK_2 (16d); dQ kernel S_1, S_2, X,
    # dQ_1, dQ_2 (12d)
    f_exec = B * H * 28 * d * npairs
    tf_alg = f_alg / (ms * 1e-3) / 1e12
    tf_exec = f_exec / (ms * 1e-3) / 1e12
    return {
        "workload": name, "ms": ms, "timing": timing, "value": round(tf_alg, 2), "unit": "TFLOP/s",
        "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "dv": 2 * d,
                   "causal": True, "window": window, "layer": layer,
                   "dtype": "bf16 in, fp32 gradients"},
        "roofline": {"bound": "mfma", "achieved": round(tf_alg, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_alg / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(name, "bwd"),
                     "executed_mfma_tflops": round(tf_exec, 2),
                     "executed_mfma_frac": round(tf_exec / PEAK_BF16_TFLOPS, 4),
                     "kernel": "bwd_dq (with the dO prologue) + bwd_dkdv + bwd_lambda (whole backward)"},
    }


def bench_train_step(da, torch, steps, warmup):
    """One V1 training step of the attention at the 4K prefill shape: the training forward (output
    plus the stash) followed by the backward for a seeded upstream gradient."""
    cfg, t = wl.make("v1_prefill_4k")
    layer = cfg["layers"][0]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    args = [to_dev(t[k], torch) for k in ("q1", "q2", "k1", "k2", "v")]
    lv = [torch.from_numpy(x).to("cuda") for x in t["lambda"][layer]]
    rng = np.random.default_rng(77)
    dy = to_dev(wl.f32_to_bf16_bits(rng.standard_normal((B, H, N, 2 * d), dtype=np.float32)), torch)
    out = torch.empty((B, H, N, 2 * d), dtype=torch.bfloat16, device="cuda")
    stash = torch.empty(da.diffattn_v1_train_stash_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    ws = torch.empty(da.diffattn_bwd_v1_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    da.diffattn_fwd_v1_train(*args, *lv, layer=layer, out=out, stash=stash)
    grads = da.diffattn_bwd_v1(*args, dy, *lv, layer=layer, stash=stash, workspace=ws)

    def fn():
        da.diffattn_fwd_v1_train(*args, *lv, layer=layer, out=out, stash=stash)
        da.diffattn_bwd_v1(*args, dy, *lv, layer=layer, stash=stash, workspace=ws, grads=grads)
    ms, timing = time_launches(fn, steps, warmup, torch)
    npairs = causal_pairs(N)
    f_alg = B * H * (8 + 16) * d * npairs      # forward 8d, backward 16d per visible pair
    f_exec = B * H * (12 + 28) * d * npairs
    tf_alg = f_alg / (ms * 1e-3) / 1e12
    tf_exec = f_exec / (ms * 1e-3) / 1e12
    return {
        "workload": "v1_train_step_4k", "ms": ms, "timing": timing, "value": round(tf_alg, 2), "unit": "TFLOP/s",
        "config": {"workload": "v1_train_step_4k", "B": B, "H": H, "N": N, "d": d, "dv": 2 * d,
                   "causal": True, "layer": layer, "dtype": "bf16 in, fp32 gradients"},
        "roofline": {"bound": "mfma", "achieved": round(tf_alg, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_alg / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("v1_train_step_4k", ("prefill", "bwd")),
                     "executed_mfma_tflops": round(tf_exec, 2),
                     "executed_mfma_frac": round(tf_exec / PEAK_BF16_TFLOPS, 4),
                     "kernel": "training forward (with stash) + backward"},
    }


# ------------------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the V1 workload)
# ------------------------------------------------------------------------------------------------

def _host_threads():
    """(cores the host reports, threads the BLAS pool uses)."""
    cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas = cores
    return cores, int(blas)


def cpu_baseline(cfg, t, budget_s):
    """The float64 oracle on whole (batch, head) slices of the V1 4K workload, for ~budget_s."""
    import oracle

    cores, blas = _host_threads()
    layer = cfg["layers"][0]
    lam = oracle.lambda_value(*t["lambda"][layer], layer)
    lam_init = oracle.lambda_init(layer)
    N, d = cfg["N"], cfg["d"]
    f32 = lambda x: wl.as_f32(x, "bf16")
    done_heads = 0
    flops = 0
    t0 = time.perf_counter()
    # whole heads, one (batch, head) after another, until the time budget is used
    for b in range(cfg["B"]):
        for h in range(cfg["H"]):
            sl = lambda x: f32(x[b:b + 1, h:h + 1])
            oracle.diff_attn_v1(sl(t["q1"]), sl(t["q2"]), sl(t["k1"]), sl(t["k2"]), sl(t["v"]),
                                lam[h:h + 1], lam_init, True, cfg["eps"])
            done_heads += 1
            flops += 8 * d * causal_pairs(N)
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas,
            "kind": "oracle", "host_cores": cores, "blas_threads": blas,
            "sample": f"{done_heads} of {cfg['B'] * cfg['H']} (batch, head) slices, all {N} causal "
                      f"rows each, of the V1 4K workload; float64 numpy oracle, {el:.1f} s, BLAS on "
                      f"{blas} threads of the host's {cores} cores"}


def cpu_baseline_long(cfg, t, budget_s):
    """The float64 oracle on seeded query rows of the 128K workload (layer 1): up to 8 blocks of 64
    uniform rows per head, head after head, until ~budget_s of oracle time have passed (the bf16
    to float64 conversion of a head's inputs, done once per head, is not timed).  Row i of a
    causal head costs 8*d*(i+1) algorithmic flops (two score rows of i+1 keys, one weighted sum
    of i+1 value rows), which is what the rate counts -- the same convention as the GPU figure."""
    import oracle

    cores, blas = _host_threads()
    layer = cfg["layers"][0]
    lam = oracle.lambda_value(*t["lambda"][layer], layer)
    lam_init = oracle.lambda_init(layer)
    N, d = cfg["N"], cfg["d"]
    rng = np.random.default_rng(4242)
    f32 = lambda x: wl.as_f32(x, "bf16")
    rows_done, flops, heads, el = 0, 0, 0, 0.0
    for h in range(cfg["H"]):
        sl = [f32(t[k][0:1, h:h + 1]) for k in ("q1", "q2", "k1", "k2", "v")]
        heads += 1
        for _ in range(8):
            rows = np.sort(rng.choice(N, size=64, replace=False))
            t0 = time.perf_counter()
            oracle.diff_attn_v1(*sl, lam[h:h + 1], lam_init, True, cfg["eps"], rows=rows)
            el += time.perf_counter() - t0
            rows_done += rows.size
            flops += int(np.sum(8 * d * (rows + 1)))
            if el > budget_s:
                break
        if el > budget_s:
            break
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas,
            "kind": "oracle", "host_cores": cores, "blas_threads": blas,
            "sample": f"{rows_done} query rows (blocks of 64 seeded uniform rows, {heads} of "
                      f"{cfg['H']} heads) of the V1 128K workload at layer {layer}, all their causal "
                      f"keys; float64 numpy oracle, {el:.1f} s of oracle time, BLAS on {blas} "
                      f"threads of the host's {cores} cores"}


# ------------------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)   # 32 steps sweep the 128K workload's layers
    ap.add_argument("--warmup", type=int, default=10)  # after SETTLE_S seconds of untimed load
    ap.add_argument("--only", choices=["long", "v1", "v2", "decode", "decode_v1", "swa", "paged", "bwd",
                                       "bwd_swa", "train"],
                    default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for "
              f"--gpus {a.gpus}); the per-GPU kernel is what one GPU shows.", file=sys.stderr)
        sys.exit(2)

    import torch

    import differential_softmax_attention_diff_amd as da

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    da.load_library()

    if a.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 3}), flush=True)
        return

    secondary = []
    head, long_inputs, v1_inputs = None, None, None
    if a.only in (None, "long"):
        print("[bench] v1 prefill, 128K context (headline)", file=sys.stderr, flush=True)
        head, long_inputs = bench_long(da, torch, a.steps, a.warmup)
        torch.cuda.empty_cache()
    if a.only in (None, "v1"):
        print("[bench] v1 prefill, 4K context", file=sys.stderr, flush=True)
        res, v1_inputs = bench_v1(da, torch, a.steps, a.warmup)
        res["value"] = round(res.pop("tflops_alg"), 2)
        res["unit"] = "TFLOP/s"
        res.pop("tflops_exec", None)
        secondary.append(res)
        torch.cuda.empty_cache()
    if a.only in (None, "v2"):
        print("[bench] v2 prefill", file=sys.stderr, flush=True)
        secondary.append(bench_v2(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "decode"):
        print("[bench] v2 decode", file=sys.stderr, flush=True)
        secondary.append(bench_decode(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "paged"):
        print("[bench] v2 decode, paged cache", file=sys.stderr, flush=True)
        secondary.append(bench_decode_paged(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "swa"):
        print("[bench] v1 prefill, sliding window", file=sys.stderr, flush=True)
        secondary.append(bench_swa(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "decode_v1"):
        print("[bench] v1 decode", file=sys.stderr, flush=True)
        secondary.append(bench_decode_v1(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "bwd"):
        print("[bench] v1 backward", file=sys.stderr, flush=True)
        secondary.append(bench_bwd_v1(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "train"):
        print("[bench] v1 training step (forward + backward)", file=sys.stderr, flush=True)
        secondary.append(bench_train_step(da, torch, a.steps, a.warmup))
        torch.cuda.empty_cache()
    if a.only in (None, "bwd_swa"):
        print("[bench] v1 backward, sliding window", file=sys.stderr, flush=True)
        cfg_w = wl.CONFIGS["v1_swa_4k"]
        secondary.append(bench_bwd_v1(da, torch, a.steps, a.warmup, window=cfg_w["window"]))
        torch.cuda.empty_cache()
    if head is None:
        head = secondary.pop(0)

    line = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": head["roofline"]["unit"],
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 activations, 6 planted needle keys per head at 128K, "
                "lambda vectors N(0, 0.1^2) per layer",
        "config": head["config"],
        "roofline": head["roofline"],
        "timing": {"settle_s": SETTLE_S, **head["timing"],
                   "policy": f"{SETTLE_S} s of untimed launches, then the warm-up steps, then the "
                             f"timed steps between HIP events on the launch stream"},
    }
    if not a.no_cpu_baseline and head["workload"] == "v1_long_128k":
        print("[bench] cpu oracle baseline (128K, sampled rows)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_long(*long_inputs, a.cpu_seconds)
    elif not a.no_cpu_baseline and head["workload"] == "v1_prefill_4k":
        print("[bench] cpu oracle baseline (4K)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(*v1_inputs, a.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    if not a.no_cpu_baseline and v1_inputs is not None and head["workload"] != "v1_prefill_4k":
        print("[bench] cpu oracle baseline (4K)", file=sys.stderr, flush=True)
        for sec in secondary:
            if sec["workload"] == "v1_prefill_4k":
                sec["cpu_baseline"] = cpu_baseline(*v1_inputs, min(a.cpu_seconds, 10.0))
    line["secondary"] = [{k: v for k, v in s.items() if k != "ms"} | {"ms_per_step": round(s["ms"], 4)}
                         for s in secondary]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

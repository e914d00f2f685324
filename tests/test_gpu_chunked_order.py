"""Workgroup order with the heads in chunks.  When the heads' streamed tiles exceed about a quarter of
the last-level cache, the V1 prefill, the V2 prefill (over KV heads) and the backward issue the heads
in chunks (multiples of 8, the last one shorter), heaviest row block first within a chunk.  The order decides only where and
when a block runs, never what it computes: a call over 12 heads at N = 32K + 5 (the prefill's
201 MB of K/V and the backward's 208 MB of tiles give chunks of 8 and 4 heads) must equal, bit for
bit, the same heads run one call each (one head: one chunk).  Per-row correctness is the parity
tests' business; this pins the chunked index arithmetic, including the short last chunk."""

import numpy as np
import pytest

import workloads as wl
from tests.helpers import dev, dev_lambda, log

pytestmark = pytest.mark.gpu

B, H, N, LAYER = 3, 4, 32768 + 5, 9


def _chunk(heads, bytes_per_head):
    """The launchers' chunk size, restated (nearest whole number of 64 MB chunks, balanced,
    rounded up to a multiple of 8)."""
    k = 64 << 20
    n = max(1, (heads * bytes_per_head + k // 2) // k)
    c = -(-heads // n)
    c = -(-c // 8) * 8
    return min(c, heads)


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


@pytest.fixture(scope="module")
def inputs():
    t = wl.make_v1(B, H, N, 64, "bf16", seed=31, layers=(LAYER,))
    x = {k: dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")}
    x["lam"] = dev_lambda(t["lambda"][LAYER])
    g = np.random.default_rng(5).standard_normal((B, H, N, 128), dtype=np.float32)
    x["dy"] = dev(wl.f32_to_bf16_bits(g))
    return x


def _head(x, b, h):
    args = [x[k][b:b + 1, h:h + 1] for k in ("q1", "q2", "k1", "k2", "v")]
    lam = [a[h:h + 1] for a in x["lam"]]
    return args, lam


def test_chunk_sizes_of_this_shape():
    assert _chunk(B * H, N * (2 * 64 + 128) * 2) == 8           # prefill: chunks of 8 and 4
    assert _chunk(B * H, N * (2 * 64 * 2 + 128 * 2 + 16)) == 8  # backward: chunks of 8 and 4
    assert _chunk(B * H, N * 2 * 128 * 2) == 8                  # V2, 12 KV heads: 8 and 4
    assert _chunk(64, 4096 * 512) == 32                         # the 4K workload: two chunks
    assert _chunk(16, 8192 * 512) == 16                         # the V2 8K workload: one chunk


def test_v1_prefill_chunked_equals_per_head(da, inputs):
    import torch

    x = inputs
    args = [x[k] for k in ("q1", "q2", "k1", "k2", "v")]
    whole = da.diffattn_fwd_v1(*args, *x["lam"], layer=LAYER)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            a, lam = _head(x, b, h)
            one = da.diffattn_fwd_v1(*a, *lam, layer=LAYER)
            torch.cuda.synchronize()
            assert torch.equal(one[0, 0], whole[b, h]), (b, h)
    log(f"  prefill over {B * H} heads at N={N} equals the per-head calls bit for bit")


def test_v1_backward_chunked_equals_per_head(da, inputs):
    import torch

    x = inputs
    args = [x[k] for k in ("q1", "q2", "k1", "k2", "v")]
    _, stash = da.diffattn_fwd_v1_train(*args, *x["lam"], layer=LAYER)
    g = da.diffattn_bwd_v1(*args, x["dy"], *x["lam"], layer=LAYER, stash=stash)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            a, lam = _head(x, b, h)
            _, st1 = da.diffattn_fwd_v1_train(*a, *lam, layer=LAYER)
            g1 = da.diffattn_bwd_v1(*a, x["dy"][b:b + 1, h:h + 1], *lam, layer=LAYER, stash=st1)
            torch.cuda.synchronize()
            # dQ, dK, dV; the lambda-vector gradients sum over every (batch, row) of a head, and the
            # per-head calls see one batch each
            for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
                assert torch.equal(g1[k][0, 0], g[k][b, h]), (k, b, h)
    log(f"  backward over {B * H} heads at N={N} equals the per-head calls bit for bit")


def test_v2_prefill_chunked_equals_per_kv_head(da):
    """V2 over B * Hkv = 12 KV heads of 2 pairs each at N = 32K + 5 (chunks of 8 and 4 KV heads)
    against one call per (batch, KV head) with its two pairs."""
    import torch

    P, Hkv = 8, 4
    ppk = P // Hkv
    t = wl.make_v2(B, P, Hkv, N, 128, "bf16", seed=41, layers=(LAYER,))
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    lam = dev_lambda(t["lambda"][LAYER])
    del t
    whole = da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], k, v, *lam, layer=LAYER)
    torch.cuda.synchronize()
    for b in range(B):
        for g in range(Hkv):
            ps = slice(g * ppk, (g + 1) * ppk)
            q1 = q[b:b + 1, 0::2][:, ps]
            q2 = q[b:b + 1, 1::2][:, ps]
            one = da.diffattn_fwd_v2(q1, q2, k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                     *[a[ps] for a in lam], layer=LAYER)
            torch.cuda.synchronize()
            assert torch.equal(one[0], whole[b, ps]), (b, g)
    log(f"  V2 prefill over {B * Hkv} KV heads at N={N} equals the per-KV-head calls bit for bit")

"""The allocation-free decode entry point (diffattn_decode_noalloc) against diffattn_decode.

Both launch the same kernels with the same split count; the only difference is where the split
partials live (the library's fixed per-GPU scratch instead of a caller workspace), so the two
outputs must be identical bit for bit -- and within the bf16 bar of the oracle.  Two calls in a
row, the second smaller than the first, check that the scratch's leftover contents from the first
call do not leak into the second; a size beyond the scratch is refused on the host.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import dev, dev_lambda, f64, log, oracle_lambda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _case(da, B, P, Hkv, L, seed, splits=0):
    import torch

    t = wl.make_decode(B, P, Hkv, L, 128, "bf16", seed=seed, layers=(24,))
    q, kc, vc = dev(t["q"]), dev(t["kcache"]), dev(t["vcache"])
    lv = dev_lambda(t["lambda"][24])
    need = da.diffattn_decode_workspace_bytes(B, P, Hkv, L, 128, splits)
    assert 0 < need <= da.DIFFATTN_DECODE_NOALLOC_MAX_BYTES
    ref_out = da.diffattn_decode(q[:, 0::2], q[:, 1::2], kc, vc, *lv, layer=24, num_splits=splits)
    out = torch.full((B, P, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    da.diffattn_decode_noalloc(q[:, 0::2], q[:, 1::2], kc, vc, *lv, layer=24, out=out,
                               num_splits=splits)
    torch.cuda.synchronize()
    return t, out, ref_out


def test_noalloc_decode_matches_workspace_decode(da):
    import torch

    # first call: the workload's head layout at a 20K-token cache, 5.3 MB of partials
    log("noalloc decode: B=40 P=16 Hkv=8 L=20000")
    t, a, b = _case(da, 40, 16, 8, 20000, seed=1700)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    lam = oracle_lambda(t["lambda"][24], 24)
    ref = oracle.diff_decode_v2(f64(t["q"][:4]), f64(t["kcache"][:4]), f64(t["vcache"][:4]), lam)
    st = compare.bf16_stats(a[:4].float().cpu().numpy(), ref, normalise=True)
    log(f"  first call: identical to diffattn_decode; oracle stats on 4 sequences {st}")
    assert compare.bf16_ok(st), st
    # second call, smaller (fewer sequences and splits, another head ratio): must not see any of
    # the first call's partials left in the scratch
    log("noalloc decode: B=3 P=4 Hkv=1 L=700, 2 splits")
    t, a, b = _case(da, 3, 4, 1, 700, seed=1701, splits=2)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    lam = oracle_lambda(t["lambda"][24], 24)
    ref = oracle.diff_decode_v2(f64(t["q"]), f64(t["kcache"]), f64(t["vcache"]), lam)
    st = compare.bf16_stats(a.float().cpu().numpy(), ref, normalise=True)
    log(f"  second call: identical; oracle stats {st}")
    assert compare.bf16_ok(st), st


def test_noalloc_decode_refuses_more_than_its_scratch(da):
    import torch

    # 64 sequences x 32 query heads x 16 splits x 130 floats = 17 MB > 16 MiB
    B, P, Hkv, L, splits = 64, 16, 8, 8192, 16
    assert da.diffattn_decode_workspace_bytes(B, P, Hkv, L, 128, splits) > da.DIFFATTN_DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((B, 2 * P, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, L, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, P, 128), dtype=torch.bfloat16, device="cuda")
    lam = torch.zeros(P, dtype=torch.float32, device="cuda")
    with pytest.raises(da.DiffAttnError) as e:
        da.diffattn_decode_noalloc(q[:, 0::2], q[:, 1::2], kc, kc, layer=24, out=out,
                                   num_splits=splits, lambda_override=lam)
    assert e.value.status == 4   # DA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.float().abs().max()) == 0.0   # nothing was enqueued

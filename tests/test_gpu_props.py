"""GPU properties of the library that do not need the oracle's values: determinism, that every
output element is written, lambda readback, strided views and host-side error codes."""

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.helpers import dev, dev_lambda, log, oracle_lambda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def test_v1_bitwise_deterministic_and_fully_written(da):
    import torch

    log("v1 determinism + NaN-poisoned output N=515")
    t = wl.make_v1(2, 3, 515, 64, "bf16", seed=1, layers=(3,))
    args = [dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    lv = dev_lambda(t["lambda"][3])
    o1 = torch.full((2, 3, 515, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    da.diffattn_fwd_v1(*args, *lv, layer=3, out=o1)
    da.diffattn_fwd_v1(*args, *lv, layer=3, out=o2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_v2_and_decode_fully_written(da):
    import torch

    log("v2/decode NaN-poisoned outputs")
    t = wl.make_v2(1, 4, 2, 77, 128, "bf16", seed=2, layers=(24,))
    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][24])
    o = torch.full((1, 4, 77, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], dev(t["k"]), dev(t["v"]), *lv, layer=24, out=o)
    ql = q[:, :, -1, :].contiguous()
    od = torch.full((1, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((da.diffattn_decode_workspace_bytes(1, 4, 2, 77, 128),), 255, dtype=torch.uint8,
                    device="cuda")  # NaN bit patterns everywhere in the workspace
    da.diffattn_decode(ql[:, 0::2], ql[:, 1::2], dev(t["k"]), dev(t["v"]), *lv, layer=24, out=od,
                       workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(od.float()).all()


def test_lambda_readback_matches_oracle(da):
    import torch

    log("lambda readback v1")
    for layer in (1, 12, 32):
        t = wl.make_v1(1, 16, 40, 64, "bf16", seed=layer, layers=(layer,))
        lam_out = torch.full((16,), float("nan"), dtype=torch.float32, device="cuda")
        da.diffattn_fwd_v1(*(dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")),
                           *dev_lambda(t["lambda"][layer]), layer=layer, lambda_out=lam_out)
        torch.cuda.synchronize()
        np.testing.assert_allclose(lam_out.cpu().numpy(), oracle_lambda(t["lambda"][layer], layer),
                                   rtol=0, atol=2e-6)


def test_v1_strided_inputs_match_contiguous(da):
    """Inputs laid out [B, N, H, d] and viewed as [B, H, N, d] give the same bits."""
    import torch

    log("v1 strided views")
    t = wl.make_v1(2, 4, 150, 64, "bf16", seed=9, layers=(4,))
    lv = dev_lambda(t["lambda"][4])
    cont = [dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    strided = [x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in cont]
    assert not strided[0].is_contiguous()
    a = da.diffattn_fwd_v1(*cont, *lv, layer=4)
    b = da.diffattn_fwd_v1(*strided, *lv, layer=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_error_codes_on_device_tensors(da):
    import torch

    log("error codes")
    x = torch.zeros(1, 1, 8, 32, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    lv = [torch.zeros(1, 32, dtype=torch.float32, device="cuda") for _ in range(4)]
    with pytest.raises(da.DiffAttnError) as e:
        da.diffattn_fwd_v1(x, x, x, x, v, *lv, layer=1)     # d = 32 is not implemented
    assert e.value.status == 3
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16, device="cuda")
    lv = [torch.zeros(1, 64, dtype=torch.float32, device="cuda") for _ in range(4)]
    with pytest.raises(da.DiffAttnError) as e:
        da.diffattn_fwd_v1(x, x, x, x, v, *lv, layer=0)     # layers are 1-based
    assert e.value.status == 2
    q = torch.zeros(1, 3, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16, device="cuda")
    lv = [torch.zeros(3, 128, dtype=torch.float32, device="cuda") for _ in range(4)]
    with pytest.raises(da.DiffAttnError) as e:
        da.diffattn_decode(q, q, kc, kc, *lv, layer=1)      # 3 pairs over 2 KV heads
    assert e.value.status == 2
    with pytest.raises(ValueError):
        da.diffattn_fwd_v1(x.cpu(), x, x, x, v, *lv, layer=1)  # no CPU path

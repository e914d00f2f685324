"""GPU properties of the library that do not need the oracle's values: determinism, that every
output element is written, lambda readback, strided views, host-side error codes and concurrent
launches on several streams."""

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


def test_concurrent_streams_match_serial(da):
    """The library keeps no mutable state between calls (the allocation-free decode's scratch
    aside): a V1 prefill, a V2 prefill, a decode step and a V1 backward launched at the same
    time on four streams (default priority), five times over, give bit for bit what each gives
    alone on the current stream."""
    import torch

    v1 = wl.make_v1(2, 4, 1000, 64, "bf16", seed=31, layers=(9,))
    v2 = wl.make_v2(1, 4, 2, 900, 128, "bf16", seed=32, layers=(24,))
    dc = wl.make_decode(8, 8, 2, 3000, 128, "bf16", seed=33, layers=(24,))
    bw = wl.make_v1(1, 2, 500, 64, "bf16", seed=34, layers=(6,))
    a1 = [dev(v1[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    l1 = dev_lambda(v1["lambda"][9])
    q2, k2, vv2 = dev(v2["q"]), dev(v2["k"]), dev(v2["v"])
    l2 = dev_lambda(v2["lambda"][24])
    qd, kc, vc = dev(dc["q"]), dev(dc["kcache"]), dev(dc["vcache"])
    ld = dev_lambda(dc["lambda"][24])
    ab = [dev(bw[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    lb = dev_lambda(bw["lambda"][6])
    rng = np.random.default_rng(35)
    dy = dev(wl.f32_to_bf16_bits(rng.standard_normal((1, 2, 500, 128)).astype(np.float32)))
    _, stash = da.diffattn_fwd_v1_train(*ab, *lb, layer=6)

    # outputs and workspaces allocated up front, one set per launch
    def buffers():
        return {
            "o1": torch.empty((2, 4, 1000, 128), dtype=torch.bfloat16, device="cuda"),
            "o2": torch.empty((1, 4, 900, 128), dtype=torch.bfloat16, device="cuda"),
            "w2": torch.empty(max(16, da.diffattn_fwd_v2_workspace_bytes(1, 2, 900, 128)), dtype=torch.uint8, device="cuda"),
            "od": torch.empty((8, 8, 128), dtype=torch.bfloat16, device="cuda"),
            "wd": torch.empty(max(16, da.diffattn_decode_workspace_bytes(8, 8, 2, 3000, 128, 0)), dtype=torch.uint8, device="cuda"),
            "wb": torch.empty(max(16, da.diffattn_bwd_v1_workspace_bytes(1, 2, 500, 64)), dtype=torch.uint8, device="cuda"),
            "g": {**{k: torch.empty((1, 2, 500, 64), dtype=torch.float32, device="cuda") for k in ("dq1", "dq2", "dk1", "dk2")},
                  "dv": torch.empty((1, 2, 500, 128), dtype=torch.float32, device="cuda"),
                  **{k: torch.empty((2, 64), dtype=torch.float32, device="cuda") for k in ("dlq1", "dlk1", "dlq2", "dlk2")}},
        }

    def launch(b, streams):
        s1, s2, s3, s4 = streams
        da.diffattn_fwd_v1(*a1, *l1, layer=9, out=b["o1"], stream=s1)
        da.diffattn_fwd_v2(q2[:, 0::2], q2[:, 1::2], k2, vv2, *l2, layer=24, out=b["o2"], workspace=b["w2"], stream=s2)
        da.diffattn_decode(qd[:, 0::2], qd[:, 1::2], kc, vc, *ld, layer=24, out=b["od"], workspace=b["wd"], stream=s3)
        da.diffattn_bwd_v1(*ab, dy, *lb, layer=6, stash=stash, workspace=b["wb"], grads=b["g"], stream=s4)

    ref = buffers()
    cur = torch.cuda.current_stream()
    launch(ref, (cur, cur, cur, cur))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(cur)  # inputs, stash and reference are complete before the concurrent launches
    for rep in range(5):
        b = buffers()
        torch.cuda.synchronize()
        launch(b, streams)
        torch.cuda.synchronize()
        same = [torch.equal(b[k], ref[k]) for k in ("o1", "o2", "od")]
        same += [torch.equal(b["g"][k], ref["g"][k]) for k in ref["g"]]
        log(f"  concurrent launch {rep}: all equal to serial: {all(same)}")
        assert all(same), same

"""Guard bands around every buffer an entry point writes.

Each output, workspace, stash and gradient buffer is carved out of a larger byte buffer whose
4 KiB before and after are filled with a canary byte; workspaces and stashes get exactly the
size the library asks for.  After the call (ragged shapes, so that tail tiles and partial blocks
run) every canary byte must be intact: a write past either end of any buffer -- which the
NaN-poisoned outputs of the other tests cannot see -- fails here.  The inputs are checked to be
unchanged as well.  One test per entry point of include/diffattn.h that writes device memory.
"""

import numpy as np
import pytest

import workloads as wl
from tests.helpers import dev, dev_lambda, log

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


class Guarded:
    """A tensor of the given shape and dtype in the middle of a canary-filled byte buffer."""

    def __init__(self, shape, dtype):
        import torch

        self.shape = tuple(shape)
        nbytes = int(np.prod(self.shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + nbytes].view(dtype).view(self.shape)

    @classmethod
    def bytes(cls, n):
        import torch

        return cls((max(int(n), 1),), torch.uint8)

    def intact(self):
        import torch

        torch.cuda.synchronize()
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes:]
        return bool((head == CANARY).all()) and bool((tail == CANARY).all())


def _inputs_unchanged(before, after):
    import torch

    return all(torch.equal(a, b) for a, b in zip(before, after))


def _check(name, bufs, inputs=None, inputs_before=None):
    bad = [k for k, g in bufs.items() if not g.intact()]
    log(f"{name}: {len(bufs)} guarded buffers, damaged: {bad}")
    assert not bad, bad
    if inputs is not None:
        assert _inputs_unchanged(inputs_before, inputs), f"{name} modified an input"


@pytest.mark.parametrize("window", [0, 45])
def test_guard_v1_bf16(da, window):
    import torch

    B, H, N, layer = 2, 3, 201, 12
    t = wl.make_v1(B, H, N, 64, "bf16", seed=1600, layers=(layer,))
    ins = [dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    before = [x.clone() for x in ins]
    out = Guarded((B, H, N, 128), torch.bfloat16)
    lam_out = Guarded((H,), torch.float32)
    da.diffattn_fwd_v1(*ins, *dev_lambda(t["lambda"][layer]), layer=layer, out=out.t, window=window,
                       lambda_out=lam_out.t)
    _check(f"fwd_v1 window={window}", {"out": out, "lambda_out": lam_out}, ins, before)


def test_guard_v1_fp32(da):
    import torch

    B, H, N, layer = 1, 3, 77, 2
    t = wl.make_v1(B, H, N, 64, "f32", seed=1601, layers=(layer,))
    ins = [dev(t[k], "f32") for k in ("q1", "q2", "k1", "k2", "v")]
    before = [x.clone() for x in ins]
    out = Guarded((B, H, N, 128), torch.float32)
    da.diffattn_fwd_v1(*ins, *dev_lambda(t["lambda"][layer]), layer=layer, out=out.t)
    _check("fwd_v1 fp32", {"out": out}, ins, before)


@pytest.mark.parametrize("window", [0, 60])
def test_guard_v2(da, window):
    import torch

    B, P, Hkv, N = 1, 4, 2, 183
    t = wl.make_v2(B, P, Hkv, N, 128, "bf16", seed=1602, layers=(24,))
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    before = [q.clone(), k.clone(), v.clone()]
    out = Guarded((B, P, N, 128), torch.bfloat16)
    ws = Guarded.bytes(da.diffattn_fwd_v2_workspace_bytes(B, Hkv, N, 128))
    da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], k, v, *dev_lambda(t["lambda"][24]), layer=24,
                       out=out.t, workspace=ws.t, window=window)
    _check(f"fwd_v2 window={window}", {"out": out, "workspace": ws}, [q, k, v], before)


def test_guard_decode(da):
    import torch

    B, P, Hkv, L = 3, 4, 2, 1111
    t = wl.make_decode(B, P, Hkv, L, 128, "bf16", seed=1603, layers=(24,))
    q, kc, vc = dev(t["q"]), dev(t["kcache"]), dev(t["vcache"])
    before = [q.clone(), kc.clone(), vc.clone()]
    out = Guarded((B, P, 128), torch.bfloat16)
    ws = Guarded.bytes(da.diffattn_decode_workspace_bytes(B, P, Hkv, L, 128, 3))
    da.diffattn_decode(q[:, 0::2], q[:, 1::2], kc, vc, *dev_lambda(t["lambda"][24]), layer=24,
                       out=out.t, workspace=ws.t, num_splits=3)
    _check("decode", {"out": out, "workspace": ws}, [q, kc, vc], before)


def test_guard_decode_v1(da):
    import torch

    B, H, L = 2, 3, 999
    t = wl.make_decode_v1(B, H, L, 64, "bf16", seed=1604, layers=(12,))
    ins = [dev(t[k]) for k in ("q1", "q2", "k1cache", "k2cache", "vcache")]
    before = [x.clone() for x in ins]
    out = Guarded((B, H, 128), torch.bfloat16)
    ws = Guarded.bytes(da.diffattn_decode_v1_workspace_bytes(B, H, L, 64, 0))
    da.diffattn_decode_v1(*ins, *dev_lambda(t["lambda"][12]), layer=12, out=out.t, workspace=ws.t)
    _check("decode_v1", {"out": out, "workspace": ws}, ins, before)


def test_guard_decode_paged(da):
    import torch

    B, P, Hkv, page = 4, 4, 2, 16
    lens = np.array([37, 700, 1, 513], dtype=np.int32)
    t = wl.make_decode_paged(B, P, Hkv, 128, page, lens, "bf16", seed=1605, layers=(24,))
    q, kp, vp = dev(t["q"]), dev(t["k_pages"]), dev(t["v_pages"])
    bt = torch.from_numpy(t["block_table"]).to("cuda")
    sl = torch.from_numpy(t["seq_lens"]).to("cuda")
    before = [q.clone(), kp.clone(), vp.clone(), bt.clone(), sl.clone()]
    max_len = int(lens.max())
    out = Guarded((B, P, 128), torch.bfloat16)
    ws = Guarded.bytes(da.diffattn_decode_workspace_bytes(B, P, Hkv, max_len, 128, 0))
    da.diffattn_decode_paged(q[:, 0::2], q[:, 1::2], kp, vp, bt, sl, *dev_lambda(t["lambda"][24]),
                             layer=24, max_len=max_len, out=out.t, workspace=ws.t)
    _check("decode_paged", {"out": out, "workspace": ws}, [q, kp, vp, bt, sl], before)


@pytest.mark.parametrize("window", [0, 50])
def test_guard_train_and_backward(da, window):
    import torch

    B, H, N, d, layer = 2, 2, 157, 64, 6
    t = wl.make_v1(B, H, N, d, "bf16", seed=1606, layers=(layer,))
    ins = [dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")]
    lv = dev_lambda(t["lambda"][layer])
    rng = np.random.default_rng(3)
    dy = dev(wl.f32_to_bf16_bits(rng.standard_normal((B, H, N, 2 * d)).astype(np.float32)))
    before = [x.clone() for x in ins + [dy]]
    out = Guarded((B, H, N, 2 * d), torch.bfloat16)
    stash = Guarded.bytes(da.diffattn_v1_train_stash_bytes(B, H, N, d))
    da.diffattn_fwd_v1_train(*ins, *lv, layer=layer, out=out.t, stash=stash.t, window=window)
    _check(f"fwd_v1_train window={window}", {"out": out, "stash": stash})
    grads = {k: Guarded((B, H, N, d), torch.float32) for k in ("dq1", "dq2", "dk1", "dk2")}
    grads["dv"] = Guarded((B, H, N, 2 * d), torch.float32)
    for k in ("dlq1", "dlk1", "dlq2", "dlk2"):
        grads[k] = Guarded((H, d), torch.float32)
    ws = Guarded.bytes(da.diffattn_bwd_v1_workspace_bytes(B, H, N, d))
    da.diffattn_bwd_v1(*ins, dy, *lv, layer=layer, stash=stash.t, workspace=ws.t, window=window,
                       grads={k: g.t for k, g in grads.items()})
    _check(f"bwd_v1 window={window}", {**grads, "workspace": ws, "stash": stash}, ins + [dy], before)

"""GPU edge cases: empty inputs through every entry point, and a sequence longer than any workload.

Empty problems (a zero batch, head or pair count, or N == 0 in a prefill) are valid calls: the
library returns DA_OK before it looks at any pointer and enqueues nothing.  Empty torch tensors
carry null data pointers, so what can show a stray write is every buffer that is not empty: the
lambda readback (filled with a sentinel) and the workspace and stash (canary bytes), which must
come back untouched.

The long case runs the V1 prefill at N = 262181 (256K + 37, ragged against the 64-row blocks) with
6 heads: B * H is not a multiple of 8, so the launch takes the plain block order, not the
one-head-per-XCD grouping that the 16-head long-context workload uses.  Sampled rows -- the first,
both sides of 2^17, the last 40 and seeded ones -- are checked against the oracle.
"""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import dev, dev_lambda, f64, log, merge_stats, oracle_lambda
from tests.test_gpu_guard_bands import CANARY, GUARD

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _zeros(shape, dtype="bf16"):
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.zeros(shape, dtype=tdt, device="cuda")


def _lam(n):
    import torch

    return torch.zeros(n, dtype=torch.float32, device="cuda")


def _sentinel(n):
    import torch

    return torch.full((n,), SENTINEL, dtype=torch.float32, device="cuda")


def _canary():
    import torch

    return torch.full((2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")


def _untouched(canary=(), sentinel=()):
    import torch

    torch.cuda.synchronize()
    return all(bool((b == CANARY).all()) for b in canary) and \
        all(bool((s == SENTINEL).all()) for s in sentinel)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N", [(0, 2, 100), (2, 0, 100), (2, 3, 0)])
def test_empty_v1(da, B, H, N, dtype):
    qk = [_zeros((B, H, N, 64), dtype) for _ in range(4)]
    v = _zeros((B, H, N, 128), dtype)
    lam_out = _sentinel(H)
    windows = (0, 5) if dtype == "bf16" else (0,)
    for window in windows:
        out = da.diffattn_fwd_v1(*qk, v, layer=3, lambda_override=_lam(H), lambda_out=lam_out,
                                 window=window)
        assert out.numel() == 0
    assert _untouched(sentinel=[lam_out])
    log(f"empty V1 {dtype} B={B} H={H} N={N}: DA_OK, lambda readback untouched")


@pytest.mark.parametrize("B,P,N", [(0, 2, 64), (1, 0, 64), (2, 2, 0)])
def test_empty_v2(da, B, P, N):
    q = _zeros((B, 2 * P, N, 128))
    k = _zeros((B, 1, N, 128))
    ws, lam_out = _canary(), _sentinel(P)
    for window in (0, 9):
        da.diffattn_fwd_v2(q[:, 0::2], q[:, 1::2], k, k, layer=24, workspace=ws,
                           lambda_override=_lam(P), lambda_out=lam_out, window=window)
    assert _untouched([ws], [lam_out])
    log(f"empty V2 B={B} P={P} N={N}: DA_OK, workspace and lambda readback untouched")


@pytest.mark.parametrize("B,P", [(0, 4), (3, 0)])
def test_empty_decodes(da, B, P):
    import torch

    q = _zeros((B, 2 * P, 128))
    kc = _zeros((B, 2, 64, 128))
    ws, lam_out = _canary(), _sentinel(P)
    da.diffattn_decode(q[:, 0::2], q[:, 1::2], kc, kc, layer=24, workspace=ws,
                       lambda_override=_lam(P), lambda_out=lam_out)
    out = _zeros((B, P, 128))
    da.diffattn_decode_noalloc(q[:, 0::2], q[:, 1::2], kc, kc, layer=24, out=out,
                               lambda_override=_lam(P), lambda_out=lam_out)
    pages = _zeros((4, 2, 16, 128))
    bt = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
    sl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    da.diffattn_decode_paged(q[:, 0::2], q[:, 1::2], pages, pages, bt, sl, layer=24, max_len=64,
                             workspace=ws, lambda_override=_lam(P), lambda_out=lam_out)
    H = P
    q1 = _zeros((B, H, 64))
    k1 = _zeros((B, H, 50, 64))
    vc = _zeros((B, H, 50, 128))
    lam1_out = _sentinel(H)
    da.diffattn_decode_v1(q1, q1, k1, k1, vc, layer=5, workspace=ws, lambda_override=_lam(H),
                          lambda_out=lam1_out)
    assert _untouched([ws], [lam_out, lam1_out])
    log(f"empty decodes B={B} P={P}: DA_OK, workspace and lambda readbacks untouched")


@pytest.mark.parametrize("window", [0, 20])
def test_empty_training(da, window):
    B, H, N = 2, 2, 0
    qk = [_zeros((B, H, N, 64)) for _ in range(4)]
    v = _zeros((B, H, N, 128))
    stash, ws, lam_out = _canary(), _canary(), _sentinel(H)
    out, _ = da.diffattn_fwd_v1_train(*qk, v, layer=4, stash=stash, lambda_override=_lam(H),
                                      lambda_out=lam_out, window=window)
    assert out.numel() == 0
    g = da.diffattn_bwd_v1(*qk, v, _zeros((B, H, N, 128)), layer=4, stash=stash, workspace=ws,
                           lambda_override=_lam(H), window=window)
    assert all(x.numel() == 0 for x in g.values())
    assert _untouched([stash, ws], [lam_out])
    log(f"empty training forward and backward window={window}: DA_OK, stash, workspace and "
        "lambda readback untouched")


@pytest.mark.timeout(600)
def test_v1_prefill_256k_plain_block_order(da):
    """V1 bf16 prefill, B=1, H=6, N=262181, causal, layer 17: sampled rows against the oracle."""
    import torch

    N, H, layer = 262144 + 37, 6, 17
    log(f"v1 bf16 B=1 H={H} N={N} layer={layer}")
    t = wl.make_v1(1, H, N, 64, "bf16", seed=2626, layers=(layer,))
    rng = np.random.default_rng(3)
    picked = set([0, 1, 63, 64, 131071, 131072] + list(range(N - 40, N)))
    while len(picked) < 64:
        picked.add(int(rng.integers(0, N)))
    rows = np.array(sorted(picked), dtype=np.int64)
    out = da.diffattn_fwd_v1(*(dev(t[k]) for k in ("q1", "q2", "k1", "k2", "v")),
                             *dev_lambda(t["lambda"][layer]), layer=layer)
    got = out[0].index_select(1, torch.from_numpy(rows).to("cuda")).float().cpu().numpy()
    del out
    lam = oracle_lambda(t["lambda"][layer], layer)
    stats = []
    for h in range(H):
        sl = [f64(t[k][:, h:h + 1]) for k in ("q1", "q2", "k1", "k2", "v")]
        ref = oracle.diff_attn_v1(*sl, lam[h:h + 1], oracle.lambda_init(layer), True, 1e-5,
                                  rows=rows)[0, 0]
        stats.append(compare.bf16_stats(got[h], ref))
    st = merge_stats(stats)
    log(f"  {H} heads x {rows.size} rows: {st}")
    assert compare.bf16_ok(st), st

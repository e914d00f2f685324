"""GPU parity of the V2 decode step on a paged KV cache with per-sequence lengths (the serving
layout) against the float64 CPU oracle, which reads each sequence's keys gathered back into a
contiguous [Hkv, L_b, D] cache.  Compared after dividing both sides by the RMS of the oracle row,
as for the contiguous V2 decode."""

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import compare
from tests.helpers import beyond_output_rounding, dev, dev_lambda, f64, log, merge_stats, oracle_lambda, parallel_map

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def _run(da, t, layer, num_splits=0, max_len=None):
    import torch

    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][layer])
    bt = torch.from_numpy(t["block_table"]).to("cuda")
    sl = torch.from_numpy(t["seq_lens"]).to("cuda")
    o = da.diffattn_decode_paged(q[:, 0::2], q[:, 1::2], dev(t["k_pages"]), dev(t["v_pages"]), bt, sl,
                                 *lv, layer=layer, num_splits=num_splits,
                                 max_len=int(t["seq_lens"].max()) if max_len is None else max_len)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _gather(t, b):
    """Contiguous [Hkv, L_b, D] K and V caches of sequence b."""
    n = int(t["seq_lens"][b])
    ps = t["k_pages"].shape[2]
    j = np.arange(n)
    pages = t["block_table"][b, j // ps]
    k = t["k_pages"][pages, :, j % ps, :].transpose(1, 0, 2)
    v = t["v_pages"][pages, :, j % ps, :].transpose(1, 0, 2)
    return k, v


def _oracle(t, layer, batches):
    lam = oracle_lambda(t["lambda"][layer], layer)
    out = []
    for b in batches:
        k, v = _gather(t, b)
        out.append(oracle.diff_decode_v2(f64(t["q"][b:b + 1]), f64(k[None]), f64(v[None]), lam)[0])
    return np.stack(out)


@pytest.mark.parametrize("P,Hkv,page,lens,splits", [
    (2, 1, 16, [1, 15, 16, 17, 1000], 0),     # G = 4, lengths around a page edge
    (16, 8, 16, [300, 5000, 2049], 0),        # the workload's head layout
    (1, 1, 64, [64, 65, 3], 3),               # G = 2, 64-key pages, fixed splits
    (8, 1, 32, [777, 128], 1),                # G = 16, unsplit
    (4, 2, 1, [5, 40], 0),                    # one key per page
])
def test_paged_decode_against_oracle(da, P, Hkv, page, lens, splits):
    log(f"paged decode P={P} Hkv={Hkv} page={page} lens={lens} splits={splits}")
    t = wl.make_decode_paged(len(lens), P, Hkv, 128, page, lens, seed=sum(lens) + page, layers=(24,))
    got = _run(da, t, 24, splits)
    ref = _oracle(t, 24, range(len(lens)))
    st = compare.bf16_stats(got, ref, normalise=True)
    log(f"  stats {st}")
    assert compare.bf16_ok(st), st


def test_paged_equals_contiguous_when_pages_are_in_order(da):
    """One sequence length for all, pages in order: the same numbers as diffattn_decode."""
    import torch

    B, P, Hkv, L, page = 2, 4, 2, 1000, 8
    t = wl.make_decode(B, P, Hkv, L, 128, "bf16", seed=17, layers=(24,))
    nb = L // page
    kp = t["kcache"].reshape(B, Hkv, nb, page, 128).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, page, 128)
    vp = t["vcache"].reshape(B, Hkv, nb, page, 128).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, page, 128)
    tp = {"q": t["q"], "k_pages": np.ascontiguousarray(kp), "v_pages": np.ascontiguousarray(vp),
          "block_table": np.arange(B * nb, dtype=np.int32).reshape(B, nb),
          "seq_lens": np.full(B, L, dtype=np.int32), "lambda": t["lambda"]}
    a = _run(da, tp, 24, num_splits=2)
    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][24])
    b = da.diffattn_decode(q[:, 0::2], q[:, 1::2], dev(t["kcache"]), dev(t["vcache"]), *lv, layer=24,
                           num_splits=2).float().cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a, b)


def test_paged_max_len_beyond_every_sequence(da):
    """A max_len above every sequence's length only adds empty splits."""
    t = wl.make_decode_paged(3, 2, 1, 128, 16, [100, 700, 33], seed=5, layers=(24,))
    a = _run(da, t, 24, max_len=700)
    t["block_table"] = np.pad(t["block_table"], ((0, 0), (0, 100)), constant_values=-1)
    b = _run(da, t, 24, max_len=t["block_table"].shape[1] * 16)   # 2304: six more, empty splits
    np.testing.assert_array_equal(a, b)


@pytest.mark.timeout(900)
def test_paged_workload_every_sequence(da):
    """The serving workload (B=64, 32 query / 8 KV heads, 16-key pages, lengths 4K..32K): every
    sequence against the oracle on its keys gathered back into a contiguous cache."""
    cfg, t = wl.make("v2_decode_paged")
    layer = cfg["layers"][0]
    log(f"paged decode workload, sum of lengths {int(t['seq_lens'].sum())}")
    got = _run(da, t, layer)
    assert np.isfinite(got).all()

    def one(b):
        ref = _oracle(t, layer, [b])
        return b, compare.bf16_stats(got[b:b + 1], ref, normalise=True), beyond_output_rounding(got[b:b + 1], ref)

    res = parallel_map(one, range(cfg["B"]))
    st = merge_stats([r[1] for r in res])
    excess = max(r[2] for r in res)
    log(f"  {cfg['B']} sequences: {st}; largest error beyond the bf16 output rounding "
        f"{excess:.2e} of the row RMS")
    assert compare.bf16_ok(st), st
    # every step before the final bf16 store runs in fp32: past the store's own rounding, what is
    # left is fp32 summation over the cache
    assert excess <= 2e-3

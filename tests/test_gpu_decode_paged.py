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


def _check(got, ref):
    """The bf16 bar on a decode output of a few sequences (reading r24): the largest error,
    normalised by the oracle row's RMS, within 2e-2, and every element within 2e-3 of that RMS
    beyond the bf16 rounding of the exact result (every step before the final store is fp32).  The
    share-within-1e-2 statistic is for populations larger than a few sequences' 128-wide rows:
    rounding the exact outputs alone can leave 2 of 1536 elements past 1e-2."""
    st = compare.bf16_stats(got, ref, normalise=True)
    ex = beyond_output_rounding(got, ref)
    log(f"  stats {st}; beyond the output rounding {ex:.2e}")
    assert st["finite"] and st["max_abs"] <= 2e-2 and ex <= 2e-3, (st, ex)


def _within_one_step(a, b):
    """Two bf16 results of the same step that differ only in fp32 summation order: every element
    within one bf16 step (2^-7 of its magnitude, the larger of the two)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b))), float(np.max(np.abs(a - b)))


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
    (4, 2, 128, [129, 640, 1], 2),            # two pages per 256-key block
    (4, 2, 256, [300, 1000, 5], 0),           # one page per block
    (2, 1, 1024, [2500, 77], 0),              # a block inside a page
    (4, 1, 16, [3000, 40, 1500], 0),          # G = 8: the per-sequence splits
    (8, 1, 16, [3000, 40, 1500], 0),          # G = 16, balanced
])
def test_paged_decode_against_oracle(da, P, Hkv, page, lens, splits):
    log(f"paged decode P={P} Hkv={Hkv} page={page} lens={lens} splits={splits}")
    t = wl.make_decode_paged(len(lens), P, Hkv, 128, page, lens, seed=sum(lens) + page, layers=(24,))
    got = _run(da, t, 24, splits)
    ref = _oracle(t, 24, range(len(lens)))
    _check(got, ref)


def test_paged_equals_contiguous_when_pages_are_in_order(da):
    """One sequence length for all, pages in order.  Unsplit (one piece per sequence and KV head
    on both paths): the same numbers as diffattn_decode, bit for bit.  With two splits the paged
    step deals all sequences' blocks evenly to its workgroups instead of splitting each sequence,
    so the pieces (and the fp32 summation order) differ from the contiguous step's: every element
    within one bf16 step."""
    import torch

    B, P, Hkv, L, page = 2, 4, 2, 1000, 8
    t = wl.make_decode(B, P, Hkv, L, 128, "bf16", seed=17, layers=(24,))
    nb = L // page
    kp = t["kcache"].reshape(B, Hkv, nb, page, 128).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, page, 128)
    vp = t["vcache"].reshape(B, Hkv, nb, page, 128).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, page, 128)
    tp = {"q": t["q"], "k_pages": np.ascontiguousarray(kp), "v_pages": np.ascontiguousarray(vp),
          "block_table": np.arange(B * nb, dtype=np.int32).reshape(B, nb),
          "seq_lens": np.full(B, L, dtype=np.int32), "lambda": t["lambda"]}
    q = dev(t["q"])
    lv = dev_lambda(t["lambda"][24])
    for splits in (1, 2):
        a = _run(da, tp, 24, num_splits=splits)
        b = da.diffattn_decode(q[:, 0::2], q[:, 1::2], dev(t["kcache"]), dev(t["vcache"]), *lv, layer=24,
                               num_splits=splits).float().cpu().numpy()
        torch.cuda.synchronize()
        if splits == 1:
            np.testing.assert_array_equal(a, b)
        else:
            _within_one_step(a, b)


def test_paged_max_len_beyond_every_sequence(da):
    """A max_len above every sequence's length only enlarges the workspace: the step still reads
    each sequence's own keys (the blocks are then dealt to more workgroups, so the result may
    differ from the tight max_len's in fp32 summation order, and both match the oracle)."""
    t = wl.make_decode_paged(3, 2, 1, 128, 16, [100, 700, 33], seed=5, layers=(24,))
    ref = _oracle(t, 24, range(3))
    a = _run(da, t, 24, max_len=700)
    t["block_table"] = np.pad(t["block_table"], ((0, 0), (0, 100)), constant_values=-1)
    b = _run(da, t, 24, max_len=t["block_table"].shape[1] * 16)   # 2304
    for x in (a, b):
        _check(x, ref)
    _within_one_step(a, b)


@pytest.mark.parametrize("lens,splits", [
    ([1] * 40, 0),                            # more workgroups than blocks: most runs are empty
    ([0, 5, 0, 0, 300, 0, 1], 0),             # empty sequences among short ones
    ([20000, 1, 1, 1, 1, 1, 1, 1], 0),        # one long sequence spread over many workgroups
    ([256, 512, 257, 255, 4096, 33], 0),      # block edges
    ([3000, 100, 5000, 700, 2000, 64], 2),    # 6 workgroups per KV head: runs cross sequences
    (list(np.random.default_rng(3).integers(0, 700, 300)), 0),  # 300 sequences: scans past 64 and 256
])
def test_paged_balanced_partition(da, lens, splits):
    """The balanced pass on uneven lengths (max_len 1000 or the longest, so that the workspace
    allows it): every sequence with keys against the oracle; a sequence of length 0 has no keys
    (its output is 0/0 and is not compared)."""
    lens = np.asarray(lens, dtype=np.int32)
    log(f"paged decode, balanced pass, lengths {lens.tolist()}, splits {splits}")
    # the generator needs a page per sequence: give empty sequences a page they never read
    t = wl.make_decode_paged(len(lens), 4, 2, 128, 16, np.maximum(lens, 1), seed=int(lens.sum()) % 1000,
                             layers=(24,))
    t["seq_lens"] = lens
    max_len = max(int(lens.max()), 1000)
    cols = -(-max_len // 16)
    t["block_table"] = np.pad(t["block_table"], ((0, 0), (0, cols - t["block_table"].shape[1])),
                              constant_values=-1)
    got = _run(da, t, 24, num_splits=splits, max_len=max_len)
    live = [b for b in range(len(lens)) if lens[b] > 0]
    ref = _oracle(t, 24, live)
    _check(got[live], ref)


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

"""HIP graph capture: the entry points enqueue kernels only (no allocation, no memset, no host
synchronisation), so a serving loop can capture them once and replay.  One graph holds a V1
prefill, a V2 decode step, the allocation-free decode step and a paged decode step on static
buffers; it is replayed four times, with new inputs (queries, caches, and for the paged cache new
per-sequence lengths) copied into those buffers eagerly between replays, and every replay is
checked bit for bit against the same calls made eagerly on the same inputs."""

import numpy as np
import pytest

import workloads as wl
from tests.helpers import dev, dev_lambda, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import differential_softmax_attention_diff_amd as mod

    mod.load_library()
    return mod


def test_graph_replays_match_eager(da):
    import torch

    B1, H1, N1, l1 = 1, 4, 700, 10
    Bd, P, Hkv, L = 6, 8, 2, 2500
    Bp, page = 5, 16
    max_len = 1200
    lens0 = np.array([1200, 37, 640, 1, 999], dtype=np.int32)

    def inputs(seed):
        v1 = wl.make_v1(B1, H1, N1, 64, "bf16", seed=seed, layers=(l1,))
        dc = wl.make_decode(Bd, P, Hkv, L, 128, "bf16", seed=seed + 1, layers=(24,))
        lens = lens0 if seed == 0 else np.random.default_rng(seed).integers(1, max_len + 1, Bp).astype(np.int32)
        # a fixed pool and table shape (the largest lengths), new values and lengths per round
        pg = wl.make_decode_paged(Bp, P, Hkv, 128, page, np.full(Bp, max_len, dtype=np.int32), "bf16",
                                  seed=seed + 2, layers=(24,))
        pg["seq_lens"] = lens
        return v1, dc, pg

    v1, dc, pg = inputs(0)
    st = {  # static device buffers the graph reads
        "v1": [dev(v1[k]) for k in ("q1", "q2", "k1", "k2", "v")],
        "q": dev(dc["q"]), "kc": dev(dc["kcache"]), "vc": dev(dc["vcache"]),
        "pq": dev(pg["q"]), "kp": dev(pg["k_pages"]), "vp": dev(pg["v_pages"]),
        "bt": torch.from_numpy(pg["block_table"]).to("cuda"), "sl": torch.from_numpy(pg["seq_lens"]).to("cuda"),
    }
    lv1 = dev_lambda(v1["lambda"][l1])
    lvd = dev_lambda(dc["lambda"][24])
    lvp = dev_lambda(pg["lambda"][24])
    outs = {
        "o1": torch.empty((B1, H1, N1, 128), dtype=torch.bfloat16, device="cuda"),
        "od": torch.empty((Bd, P, 128), dtype=torch.bfloat16, device="cuda"),
        "on": torch.empty((Bd, P, 128), dtype=torch.bfloat16, device="cuda"),
        "op": torch.empty((Bp, P, 128), dtype=torch.bfloat16, device="cuda"),
    }
    wsd = torch.empty(da.diffattn_decode_workspace_bytes(Bd, P, Hkv, L, 128, 0), dtype=torch.uint8, device="cuda")
    wsp = torch.empty(da.diffattn_decode_workspace_bytes(Bp, P, Hkv, max_len, 128, 0), dtype=torch.uint8, device="cuda")

    def calls(o):
        da.diffattn_fwd_v1(*st["v1"], *lv1, layer=l1, out=o["o1"])
        da.diffattn_decode(st["q"][:, 0::2], st["q"][:, 1::2], st["kc"], st["vc"], *lvd, layer=24, out=o["od"],
                           workspace=wsd)
        da.diffattn_decode_noalloc(st["q"][:, 0::2], st["q"][:, 1::2], st["kc"], st["vc"], *lvd, layer=24,
                                   out=o["on"])
        da.diffattn_decode_paged(st["pq"][:, 0::2], st["pq"][:, 1::2], st["kp"], st["vp"], st["bt"], st["sl"],
                                 *lvp, layer=24, max_len=max_len, out=o["op"], workspace=wsp)

    # warm up eagerly (library load, the allocation-free decode's one-time scratch lookup)
    calls(outs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            calls(outs)
    torch.cuda.synchronize()

    for rnd in range(4):
        v1, dc, pg = inputs(100 * rnd)
        for i, k in enumerate(("q1", "q2", "k1", "k2", "v")):
            st["v1"][i].copy_(dev(v1[k]))
        st["q"].copy_(dev(dc["q"]))
        st["kc"].copy_(dev(dc["kcache"]))
        st["vc"].copy_(dev(dc["vcache"]))
        st["pq"].copy_(dev(pg["q"]))
        st["kp"].copy_(dev(pg["k_pages"]))
        st["vp"].copy_(dev(pg["v_pages"]))
        st["bt"].copy_(torch.from_numpy(pg["block_table"]).to("cuda"))
        st["sl"].copy_(torch.from_numpy(pg["seq_lens"]).to("cuda"))
        for o in outs.values():
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = {k: torch.empty_like(v) for k, v in outs.items()}
        calls(eager)
        torch.cuda.synchronize()
        same = {k: bool(torch.equal(outs[k], eager[k])) for k in outs}
        log(f"  replay {rnd} (paged lengths {[int(x) for x in pg['seq_lens']]}): equal to eager {same}")
        assert all(same.values()), same
        assert torch.equal(outs["on"], outs["od"])  # the allocation-free decode equals the workspace one

"""CPU checks of the seeded synthetic workload generators (no method arithmetic lives there)."""

import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s
                        for s in (1e-3, 1.0, 37.0)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_deterministic_and_thread_independent(monkeypatch):
    a = wl.normal_tensor(7, "q1", (2, 3, 5, 8), "bf16")
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    b = wl.normal_tensor(7, "q1", (2, 3, 5, 8), "bf16")
    np.testing.assert_array_equal(a, b)
    c = wl.normal_tensor(8, "q1", (2, 3, 5, 8), "bf16")
    assert not np.array_equal(a, c)
    # a slice does not depend on the other slices' sizes
    big = wl.normal_tensor(7, "q1", (3, 4, 5, 8), "bf16")
    np.testing.assert_array_equal(big[:2, :3], a)


def test_value_distribution():
    x = wl.as_f32(wl.normal_tensor(1, "v", (1, 4, 4096, 64), "bf16"), "bf16")
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1) < 0.01
    lv = wl.lambda_vectors(1, 16, 64, 3)
    assert len(lv) == 4 and lv[0].shape == (16, 64)
    assert abs(float(np.std(np.stack(lv))) - 0.1) < 0.01
    # per-layer vectors differ
    assert not np.array_equal(lv[0], wl.lambda_vectors(1, 16, 64, 4)[0])


def test_needles_planted_in_branch_one_only():
    t = wl.make_v1(1, 2, 300, 64, "bf16", seed=5, needles=6)
    pos = t["needle_pos"]
    assert pos.shape == (1, 2, 6)
    for h in range(2):
        assert len(set(pos[0, h].tolist())) == 6 and pos[0, h].max() < 299
        q = wl.as_f32(t["q1"][0, h, -1], "bf16").astype(np.float64)
        for j in pos[0, h]:
            k = wl.as_f32(t["k1"][0, h, j], "bf16").astype(np.float64)
            assert abs(np.linalg.norm(k) - 4.0) < 0.05
            assert np.dot(k, q) / (np.linalg.norm(k) * np.linalg.norm(q)) > 0.999
    fresh = wl.make_v1(1, 2, 300, 64, "bf16", seed=5)
    np.testing.assert_array_equal(fresh["k2"], t["k2"])
    np.testing.assert_array_equal(fresh["q1"], t["q1"])


def test_config_table_shapes():
    cfg, t = wl.make("v1_fp32_small")
    assert t["q1"].shape == (1, 2, 128, 64) and t["q1"].dtype == np.float32
    assert t["v"].shape == (1, 2, 128, 128)
    assert sorted(t["lambda"]) == [1, 2, 3, 4]
    cfg, t = wl.make("v2_prefill_8k", N=64)
    assert t["q"].shape == (2, 32, 64, 128) and t["k"].shape == (2, 8, 64, 128)
    cfg, t = wl.make("v2_decode_32k", B=2, L=50)
    assert t["q"].shape == (2, 32, 128) and t["kcache"].shape == (2, 8, 50, 128)

"""The seeded input generator: determinism, bfloat16 rounding, recipe properties."""
import numpy as np
import torch

import synth


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  1e-38, 3.0e38], dtype=np.float32)])
    ours = synth.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_bits_roundtrip():
    x = synth.bf16_round(np.random.default_rng(1).standard_normal(1000).astype(np.float32))
    bits = synth.bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, x)


def test_deterministic_and_prefix_stable():
    a = synth.make_qkv(3, 2, 6, 5, 8, workload_id=9)
    b = synth.make_qkv(3, 2, 6, 5, 8, workload_id=9)
    c = synth.make_qkv(2, 2, 6, 5, 8, workload_id=9)
    for x, y, z in zip(a, b, c):
        assert x.shape == (3, 2, 30, 8) and x.dtype == np.float32
        assert np.array_equal(x, y)
        assert np.array_equal(x[:2], z)
    assert not np.array_equal(a[0], a[1])


def test_workload_table():
    names = [w["name"] for w in synth.WORKLOADS]
    assert names == ["tiny-fp32", "deit-t", "deit-s", "hires-3136", "long-16k", "ade-1024",
                     "ade-1600", "seq-64k", "seq-256k"]
    for w in synth.WORKLOADS:
        assert (w["grid_h"] * w["grid_w"]) >= w["k"] >= 1
        assert w["d"] == 64
    # the segmentation grids take m = k = 49; the 1-D sequences m * k = N / 4
    for name, n in [("ade-1024", 1024), ("ade-1600", 1600)]:
        w = synth.workload(name)
        assert w["grid_h"] * w["grid_w"] == n and w["m_h"] * w["m_w"] == w["k"] == 49
    for name in ("seq-64k", "seq-256k"):
        w = synth.workload(name)
        N = w["grid_h"] * w["grid_w"]
        assert w["grid_h"] == 1 and w["m_h"] == 1 and w["m_w"] * w["k"] * 4 == N
        assert w["H"] * w["d"] == 128


def test_tiny_is_plain_fp32_normal():
    Q, K, V = synth.workload_inputs("tiny-fp32")
    assert Q.shape == (1, 1, 196, 64)
    assert np.any(Q.view(np.uint32) & 0xFFFF)   # not bf16-rounded
    assert abs(Q.std() - 1) < 0.05


def test_smooth_component_is_spatially_coherent():
    Q, _, _ = synth.make_qkv(2, 2, 14, 14, 64, workload_id=1)
    g = Q.reshape(2, 2, 14, 14, 64).astype(np.float64)
    # neighbouring tokens share the smooth term: their correlation is about 2/3
    a, b = g[:, :, :, :-1, :].ravel(), g[:, :, :, 1:, :].ravel()
    r = np.corrcoef(a, b)[0, 1]
    assert 0.4 < r < 0.8, r
    assert abs(g.var() - 3.0) < 0.4   # N(0,1) noise + four unit sinusoids (variance 2)
    assert np.all((Q.view(np.uint32) & 0xFFFF) == 0)

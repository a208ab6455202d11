"""Host-side checks of the seeded synthetic input generators."""
import numpy as np

import workloads as wl


def test_bf16_rounding_of_draws_is_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3e38], dtype=np.float32)
    got = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(f))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2**-6 and got[3] == -2.5


def test_top2_routing_bookkeeping():
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((64, 8))
    bias = rng.standard_normal(8)
    split, token, probs = wl.route_top2(logits, bias)
    assert split.sum() == 128 and split.max() <= 64
    # every token appears twice, and its two weights sum to 1
    assert np.array_equal(np.bincount(token, minlength=64), np.full(64, 2))
    s = np.zeros(64)
    np.add.at(s, token, probs.astype(np.float64))
    np.testing.assert_allclose(s, 1.0, rtol=1e-6)
    # rows grouped by expert, tokens ascending within an expert
    off = np.concatenate([[0], np.cumsum(split)])
    for e in range(8):
        t = token[off[e]:off[e + 1]]
        assert np.all(np.diff(t) > 0)


def test_tiny_workload_has_empty_middle_expert():
    d = wl.make_mlp_inputs(wl.WORKLOADS["tiny_moe_fwd"])
    assert d["split_sizes"][1] == 0 and d["split_sizes"].sum() == 512
    assert d["x"].shape == (512, 256) and d["w1"].shape == (4, 1024, 256)
    assert d["w2"].shape == (4, 256, 512) and d["probs"].dtype == np.float32


def test_quantize_tensor_has_zero_tiles_and_outliers():
    x = wl.quantize_tensor_c2(rows=1024, cols=512)
    v = wl.f32_from_bf16_bits(x)
    t = v.reshape(32, 32, 16, 32)
    assert np.any(np.all(t == 0, axis=(1, 3)))
    assert np.abs(v).max() > 1000

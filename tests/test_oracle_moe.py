"""Pins of the oracle's token dispatch and combine (readings R12, R13):
a hand-worked example, agreement with the routing bookkeeping of the input
generator (an independent formulation: one stable argsort of expert*T+token),
the closed form combine(dispatch(x)) = k*x, and dropped out-of-range experts."""
import numpy as np

import oracle as orc
import workloads as wl


def test_dispatch_hand_worked():
    # tokens 0..2 pick experts (2,0), (0,1), (2,1): expert 0 gets tokens 0, 1;
    # expert 1 gets 1, 2; expert 2 gets 0, 2
    idx = np.array([[2, 0], [0, 1], [2, 1]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [0.6, 0.4], [0.9, 0.1]], dtype=np.float32)
    x = np.arange(6, dtype=np.float64).reshape(3, 2)
    d = orc.moe_dispatch(x, idx, w, 3)
    assert d["counts"].tolist() == [2, 2, 2]
    assert d["row_token"].tolist() == [0, 1, 1, 2, 0, 2]
    assert d["perm"].tolist() == [[4, 0], [1, 2], [5, 3]]
    assert np.allclose(d["probs_perm"], [0.3, 0.6, 0.4, 0.1, 0.7, 0.9])
    assert np.array_equal(d["x_perm"], x[[0, 1, 1, 2, 0, 2]])


def test_dispatch_matches_route_top2_bookkeeping():
    rng = np.random.default_rng(40)
    T, E = 300, 8
    logits = rng.standard_normal((T, E))
    bias = rng.standard_normal(E)
    split, token_of_row, probs = wl.route_top2(logits, bias)
    idx, w = wl.top2_picks(logits, bias)
    d = orc.moe_dispatch(np.arange(T)[:, None], idx, w, E)
    assert np.array_equal(d["counts"], split)
    assert np.array_equal(d["row_token"], token_of_row)
    assert np.array_equal(d["probs_perm"], probs)


def test_combine_of_dispatch_is_k_times_x():
    rng = np.random.default_rng(41)
    T, H, E = 64, 32, 5
    x_bits = wl.normal_bf16(rng, (T, H), 1.0)
    idx = np.stack([rng.permutation(E)[:2] for _ in range(T)]).astype(np.int32)
    d = orc.moe_dispatch(x_bits, idx, None, E)
    y = orc.moe_combine(d["x_perm"], d["perm"])
    assert np.array_equal(y, 2.0 * orc.bf16_bits_to_f64(x_bits))     # doubling is exact in bf16


def test_out_of_range_experts_are_dropped():
    idx = np.array([[0, 3], [-1, 1], [1, 0]], dtype=np.int32)      # E = 2: 3 and -1 dropped
    d = orc.moe_dispatch(np.zeros((3, 1)), idx, None, 2)
    assert d["counts"].tolist() == [2, 2]
    assert d["perm"].tolist() == [[0, -1], [-1, 2], [3, 1]]
    y = orc.moe_combine(np.full((4, 1), 0x3F80, dtype=np.uint16), d["perm"])   # 1.0 in bf16
    assert y[:, 0].tolist() == [1.0, 1.0, 2.0]

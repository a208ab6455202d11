"""Pins of the oracle's grouped GEMM and fused MLP (forward and backward)
against brute force, exact-integer cases, closed forms, a library routine
(torch autograd in float64 on the unquantized MLP) and finite differences.

GroupedLinear over split_sizes, GroupedLinear -> ScaledSwiGLU -> GroupedLinear
with routing-weight scaling and its backward: "Efficient MoE training for
biological foundation models", Key technical approaches items 1 and 3."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl


# ---------------------------------------------------------------------------
# grouped GEMM

def _triple_loop(A, B):
    M, K = A.shape
    N = B.shape[0]
    C = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(A[i, k]) * float(B[j, k])
            C[i][j] = s
    return np.array(C)


def test_gemm_group_m_vs_triple_loop():
    rng = np.random.default_rng(10)
    sizes = [3, 0, 5]
    aq, as_ = wl.random_mx_operand(rng, 8, 64)
    bq = np.zeros((3, 4, 64), np.uint8)
    bs = np.zeros((3, 4, 2), np.uint8)
    for g in range(3):
        bq[g], bs[g] = wl.random_mx_operand(rng, 4, 64)
    C = orc.gemm_group_m(aq, as_, bq, bs, sizes)
    # brute force: decode each code by table lookup of its magnitude, scale, triple loop
    A = orc.e4m3_value(aq) * np.repeat(orc.e8m0_value(as_), 32, axis=1)
    want = np.zeros((8, 4))
    want[0:3] = _triple_loop(A[0:3], orc.e4m3_value(bq[0]) * np.repeat(orc.e8m0_value(bs[0]), 32, axis=1))
    want[3:8] = _triple_loop(A[3:8], orc.e4m3_value(bq[2]) * np.repeat(orc.e8m0_value(bs[2]), 32, axis=1))
    np.testing.assert_allclose(C, want, rtol=1e-12, atol=0)


def test_gemm_integer_codes_exact():
    """Codes encoding small integers with unit scales: every product and sum is an
    exact integer, so the result is known exactly."""
    rng = np.random.default_rng(11)
    ints = rng.integers(-16, 17, size=(40, 256))
    ints_b = rng.integers(-16, 17, size=(2, 24, 256))
    enc = lambda v: orc.e4m3_encode(v.astype(np.float64))
    aq, bq = enc(ints), enc(ints_b)
    as_ = np.full((40, 8), 127, np.uint8)
    bs = np.full((2, 24, 8), 127, np.uint8)
    C = orc.gemm_group_m(aq, as_, bq, bs, [15, 25])
    want = np.concatenate([ints[:15] @ ints_b[0].T, ints[15:] @ ints_b[1].T])
    assert np.array_equal(C, want.astype(np.float64))


def test_gemm_group_k_is_loop_of_dense_and_zero_group():
    rng = np.random.default_rng(12)
    sizes = np.array([40, 0, 7, 64])
    P = orc.padded_sizes(sizes)
    x = rng.standard_normal((sizes.sum(), 48))
    y = rng.standard_normal((sizes.sum(), 80))
    aq, as_ = orc.quantize_colwise(x, sizes)       # [48, sum P]
    bq, bs = orc.quantize_colwise(y, sizes)        # [80, sum P]
    C = orc.gemm_group_k(aq, as_, bq, bs, sizes)
    assert C.shape == (4, 48, 80)
    assert np.all(C[1] == 0)
    r0 = 0
    for g, m in enumerate(sizes):
        if m:
            xa = orc.dequantize_rowwise(*orc.quantize_colwise(x[r0:r0 + m]))[:, :m]
            yb = orc.dequantize_rowwise(*orc.quantize_colwise(y[r0:r0 + m]))[:, :m]
            np.testing.assert_allclose(C[g], xa @ yb.T, rtol=1e-12, atol=1e-12)
        r0 += m


# ---------------------------------------------------------------------------
# fused MLP forward

def _torch_mlp(x, p, w1, w2, split, F):
    """Unquantized grouped MLP with torch float64 ops (library reference)."""
    out = []
    r0 = 0
    for e, m in enumerate(split):
        xe = x[r0:r0 + m]
        h = xe @ w1[e].T
        a = p[r0:r0 + m, None] * torch.nn.functional.silu(h[:, :F]) * h[:, F:]
        out.append(a @ w2[e].T)
        r0 += m
    return torch.cat(out)


def _case(seed=20, E=3, H=64, F=96, split=(37, 0, 50)):
    return wl.small_mlp_case(seed, E, H, F, split)


def test_unquantized_forward_matches_torch():
    c = _case()
    F = c["w1"].shape[1] // 2
    got = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], quantize=False)
    t = lambda a: torch.tensor(orc.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64))
    want = _torch_mlp(t(c["x"]), t(c["probs"]), t(c["w1"]), t(c["w2"]), c["split_sizes"].tolist(), F)
    np.testing.assert_allclose(got["y_exact"], want.numpy(), rtol=1e-10, atol=1e-14)


def test_forward_identity_weights_closed_form():
    """W1 = [I; 2I], W2 = I: H1 = [X, 2X], A = w*silu(X)*2X, Y = quantized A."""
    rng = np.random.default_rng(21)
    H = F = 64
    R = 40
    x = rng.integers(-8, 9, size=(R, H)).astype(np.float64) / 4.0
    I = np.eye(F)
    w1 = np.concatenate([I, 2 * I])[None].astype(np.float64)
    w2 = I[None]
    p = rng.uniform(0.1, 1.0, R)
    got = orc.mlp_forward(x, p, w1, w2, [R])
    import math
    A = np.array([[p[r] * (x[r, j] / (1.0 + math.exp(-x[r, j]))) * 2 * x[r, j]
                   for j in range(F)] for r in range(R)])
    # inputs x/4 in [-2, 2] are exact in MXFP8 (small dyadics), identity weights too,
    # so H1 is exact and Y is the rowwise quantization of A
    np.testing.assert_array_equal(got["h1"], np.concatenate([x, 2 * x], axis=1))
    np.testing.assert_allclose(got["a"], A, rtol=1e-13, atol=1e-300)
    qa = orc.dequantize_rowwise(*orc.quantize_rowwise(A))
    np.testing.assert_array_equal(got["y"], orc.round_to_bf16(qa))


def test_grouped_forward_is_loop_of_single_expert_calls():
    c = _case()
    split = c["split_sizes"]
    got = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split)
    r0 = 0
    for e, m in enumerate(split.tolist()):
        if m:
            one = orc.mlp_forward(c["x"][r0:r0 + m], c["probs"][r0:r0 + m],
                                  c["w1"][e:e + 1], c["w2"][e:e + 1], [m])
            np.testing.assert_array_equal(got["y"][r0:r0 + m], one["y"])
        r0 += m


def test_routing_weight_power_of_two_shifts_scales_only():
    c = _case(split=(64,), E=1)
    one = orc.mlp_forward(c["x"], np.ones(64), c["w1"], c["w2"], [64])
    four = orc.mlp_forward(c["x"], np.full(64, 4.0), c["w1"], c["w2"], [64])
    q1, s1 = orc.quantize_rowwise(one["a"])
    q4, s4 = orc.quantize_rowwise(four["a"])
    assert np.array_equal(q1, q4)
    assert np.array_equal(s4.astype(int), s1.astype(int) + 2)
    np.testing.assert_array_equal(four["y"], 4 * one["y"])
    zero = orc.mlp_forward(c["x"], np.zeros(64), c["w1"], c["w2"], [64])
    assert np.all(zero["y"] == 0)


def test_row_permutation_within_expert():
    c = _case(split=(50, 30), E=2)
    got = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], [50, 30])
    perm = np.concatenate([np.random.default_rng(1).permutation(50), 50 + np.arange(30)])
    got2 = orc.mlp_forward(c["x"][perm], c["probs"][perm], c["w1"], c["w2"], [50, 30])
    np.testing.assert_array_equal(got2["y"], got["y"][perm])


def test_forward_rows_matches_full():
    c = _case()
    full = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    rows = np.array([0, 5, 36, 37, 60, 86])
    part = orc.mlp_forward_rows(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], rows)
    np.testing.assert_array_equal(part["y"], full["y"][rows])


# ---------------------------------------------------------------------------
# backward

def _torch_grads(c):
    F = c["w1"].shape[1] // 2
    t = lambda a: torch.tensor(orc.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64),
                               requires_grad=True)
    x, p, w1, w2 = t(c["x"]), t(c["probs"]), t(c["w1"]), t(c["w2"])
    y = _torch_mlp(x, p, w1, w2, c["split_sizes"].tolist(), F)
    dy = torch.tensor(orc.bf16_bits_to_f64(c["dy"]))
    (y * dy).sum().backward()
    return dict(dx=x.grad.numpy(), dprobs=p.grad.numpy(), dw1=w1.grad.numpy(), dw2=w2.grad.numpy())


def test_unquantized_backward_matches_torch_autograd():
    c = _case()
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], quantize=False)
    got = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], fwd,
                           quantize=False)
    want = _torch_grads(c)
    np.testing.assert_allclose(got["dx_exact"], want["dx"], rtol=1e-9, atol=1e-16)
    np.testing.assert_allclose(got["dprobs"], want["dprobs"], rtol=1e-9, atol=1e-16)
    np.testing.assert_allclose(got["dw1"], want["dw1"], rtol=1e-9, atol=1e-16)
    np.testing.assert_allclose(got["dw2"], want["dw2"], rtol=1e-9, atol=1e-16)


def test_unquantized_backward_finite_differences():
    c = _case(E=2, H=32, F=32, split=(9, 7))
    x = orc.bf16_bits_to_f64(c["x"])
    w1 = orc.bf16_bits_to_f64(c["w1"])
    w2 = orc.bf16_bits_to_f64(c["w2"])
    p = c["probs"].astype(np.float64)
    dy = orc.bf16_bits_to_f64(c["dy"])
    split = c["split_sizes"]
    loss = lambda x_, p_, w1_, w2_: float(np.sum(
        orc.mlp_forward(x_, p_, w1_, w2_, split, quantize=False)["y_exact"] * dy))
    fwd = orc.mlp_forward(x, p, w1, w2, split, quantize=False)
    g = orc.mlp_backward(x, p, w1, w2, split, dy, fwd, quantize=False)
    h = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in (("x", x, g["dx_exact"]), ("p", p, g["dprobs"]),
                            ("w1", w1, g["dw1"]), ("w2", w2, g["dw2"])):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = dict(x_=x, p_=p, w1_=w1, w2_=w2)
            args_m = dict(args_p)
            key = {"x": "x_", "p": "p_", "w1": "w1_", "w2": "w2_"}[name]
            args_p[key], args_m[key] = ap, am
            fd = (loss(**args_p) - loss(**args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def test_quantized_backward_close_to_unquantized():
    """Straight-through MXFP8 gradients track the exact gradients to within
    quantization noise; a transposed or mis-grouped operand would not."""
    c = _case(E=3, H=128, F=128, split=(70, 0, 90))
    q = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    gq = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], q)
    e = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], quantize=False)
    ge = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], e,
                          quantize=False)
    assert _rel(q["y_exact"], e["y_exact"]) < 0.1
    for k in ("dx_exact", "dprobs", "dw1", "dw2"):
        assert _rel(gq[k], ge[k]) < 0.15, k
    # a zero-row expert has a zero weight gradient
    assert np.all(gq["dw1"][1] == 0) and np.all(gq["dw2"][1] == 0)


def test_dprobs_identity_and_accumulate():
    c = _case()
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    g = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], fwd)
    # sum_r w_r dprobs_r = sum dA * A with A = w * silu(g) * u (bf16 H1 in the bwd)
    F = c["w1"].shape[1] // 2
    h1 = fwd["h1_bf16"]
    w = c["probs"].astype(np.float64)
    A_b = w[:, None] * orc.silu(h1[:, :F]) * h1[:, F:]
    lhs = np.sum(w * g["dprobs"])
    rhs = np.sum(g["da"] * A_b)
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(rhs))
    base1 = np.full(c["w1"].shape, 0.25)
    base2 = np.full(c["w2"].shape, -0.5)
    g2 = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], fwd,
                          dw1_in=base1, dw2_in=base2)
    np.testing.assert_allclose(g2["dw1"], g["dw1"] + base1, rtol=0, atol=1e-15)
    assert np.all(g2["dw1"][1] == 0.25) and np.all(g2["dw2"][1] == -0.5)   # empty expert untouched


def test_sampled_backward_matches_full():
    c = _case()
    split = c["split_sizes"]
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split)
    g = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], fwd)
    rows = np.array([1, 36, 37, 80, 86])
    part = orc.mlp_backward_rows(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], rows)
    np.testing.assert_allclose(part["dx"], g["dx"][rows], rtol=0, atol=0)
    np.testing.assert_allclose(part["dprobs"], g["dprobs"][rows], rtol=1e-12, atol=1e-18)
    i1 = np.array([[0, 3], [100, 63], [191, 0]])
    i2 = np.array([[5, 7], [63, 95]])
    d1, d2 = orc.mlp_backward_wgrad_entries(c["x"], c["probs"], c["w1"], c["w2"], split,
                                            c["dy"], 2, i1, i2)
    np.testing.assert_allclose(d1, g["dw1"][2][i1[:, 0], i1[:, 1]], rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(d2, g["dw2"][2][i2[:, 0], i2[:, 1]], rtol=1e-12, atol=1e-18)

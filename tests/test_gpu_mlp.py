"""GPU parity of the fused grouped MLP (grouped_mlp_fwd / grouped_mlp_bwd)
against the oracle: GroupedLinear -> ScaledSwiGLU -> GroupedLinear with
routing-weight scaling and its backward ("Efficient MoE training for
biological foundation models", Key technical approaches item 3).

Bar: normwise relative error <= 2e-2 for Y, dX, dW1, dW2 and dprobs, both
over the whole output and per expert with rows. Requantized intermediates
(A, dH1) are computed from fp32 on the GPU and fp64 in the oracle, so a code
can differ by one step where the two straddle a rounding boundary."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, rel_norm, to_np

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _check_rows(got, want, split, what):
    assert rel_norm(got, want) <= TOL, what
    r0 = 0
    for e, m in enumerate(split):
        if m:
            err = rel_norm(got[r0:r0 + m], want[r0:r0 + m])
            assert err <= TOL, f"{what} expert {e}: {err}"
        r0 += m


def _run(mx, c, training=True, probs=True):
    x, w1, w2 = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"])
    p = dev_f32(c["probs"]) if probs else None
    y, st = mx.grouped_mlp_fwd(x, p, w1, w2, c["split_sizes"].tolist(), training=training)
    torch.cuda.synchronize()
    return y, st, p


CASES = {
    "ragged4": dict(seed=30, E=4, H=256, F=384, split=(300, 0, 17, 200)),
    "two_tiles_ffn": dict(seed=31, E=3, H=512, F=768, split=(257, 33, 190)),
    "dense_one_expert": dict(seed=32, E=1, H=256, F=512, split=(384,)),
    # GEMM2 (K = F = 1024, 8 k-steps) and dgrad1 (K = 2F) take the split-K
    # tail path: fewer tiles than half the CUs, each split into k-step parts
    "split_k_tail": dict(seed=33, E=2, H=256, F=1024, split=(300, 100)),
    # many small groups around the 32-, 64- and 128-row boundaries (k-tiled
    # scale words shared by a group's last rows, waves with no rows of their
    # group) at the smallest hidden size
    "many_small": dict(seed=34, E=12, H=128, F=256,
                       split=(1, 31, 32, 33, 0, 64, 95, 96, 97, 127, 128, 129)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward(gpu_lib, name):
    k = CASES[name]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    y, _, _ = _run(gpu_lib, c, training=False)
    want = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    _check_rows(to_np(y), want["y"], k["split"], "y")


def test_forward_tiny_workload(gpu_lib):
    """The tiny MoE workload (256 tokens, top-2 of 4 experts, one expert empty)."""
    c = wl.make_mlp_inputs(wl.WORKLOADS["tiny_moe_fwd"])
    y, _, _ = _run(gpu_lib, c, training=False)
    want = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    _check_rows(to_np(y), want["y"], c["split_sizes"].tolist(), "y")


def test_forward_training_matches_inference(gpu_lib):
    k = CASES["ragged4"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    y1, _, _ = _run(gpu_lib, c, training=False)
    y2, st, _ = _run(gpu_lib, c, training=True)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert st is not None


def test_forward_routing_weight_zero_and_pow2(gpu_lib):
    k = CASES["ragged4"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"], probs="one")
    y1, _, _ = _run(gpu_lib, c, training=False)
    c4 = dict(c, probs=np.full_like(c["probs"], 4.0))
    y4, _, _ = _run(gpu_lib, c4, training=False)
    # w = 2^k only shifts A's scales, so Y scales exactly
    assert torch.equal((y1.float() * 4).view(torch.int32), y4.float().view(torch.int32))
    c0 = dict(c, probs=np.zeros_like(c["probs"]))
    y0, _, _ = _run(gpu_lib, c0, training=False)
    assert torch.count_nonzero(y0.float()) == 0
    # probs=None means weight 1
    yn, _, _ = _run(gpu_lib, c, training=False, probs=False)
    assert torch.equal(yn.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("name", ["ragged4", "two_tiles_ffn", "dense_one_expert", "split_k_tail", "many_small"])
def test_backward(gpu_lib, name):
    k = CASES[name]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    y, st, p = _run(gpu_lib, c, training=True)
    dy = dev_bf16(c["dy"])
    dx, dprobs, dw1, dw2 = gpu_lib.grouped_mlp_bwd(dy, p, st)
    torch.cuda.synchronize()
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    want = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], fwd)
    split = list(k["split"])
    _check_rows(to_np(dx), want["dx"], split, "dx")
    _check_rows(to_np(dprobs), want["dprobs"], split, "dprobs")
    g1, g2 = to_np(dw1), to_np(dw2)
    assert rel_norm(g1, want["dw1"]) <= TOL and rel_norm(g2, want["dw2"]) <= TOL
    for e, m in enumerate(split):
        if m:
            assert rel_norm(g1[e], want["dw1"][e]) <= TOL, f"dw1 expert {e}"
            assert rel_norm(g2[e], want["dw2"][e]) <= TOL, f"dw2 expert {e}"
        else:
            assert np.all(g1[e] == 0) and np.all(g2[e] == 0)


def test_backward_accumulates_into_main_grad(gpu_lib):
    k = CASES["ragged4"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    _, st, p = _run(gpu_lib, c, training=True)
    dy = dev_bf16(c["dy"])
    E, H, F = k["E"], k["H"], k["F"]
    base1 = torch.full((E, 2 * F, H), 0.25, device="cuda")
    base2 = torch.full((E, H, F), -0.5, device="cuda")
    _, _, dw1, dw2 = gpu_lib.grouped_mlp_bwd(dy, p, st, dw1=base1.clone(), dw2=base2.clone(),
                                             accumulate=True)
    _, _, f1, f2 = gpu_lib.grouped_mlp_bwd(dy, p, st)
    torch.cuda.synchronize()
    assert torch.allclose(dw1, f1 + base1, rtol=0, atol=1e-6)
    assert torch.allclose(dw2, f2 + base2, rtol=0, atol=1e-6)
    assert torch.all(dw1[1] == 0.25) and torch.all(dw2[1] == -0.5)    # empty expert untouched


def test_autograd_function(gpu_lib):
    k = CASES["two_tiles_ffn"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    x = dev_bf16(c["x"]).requires_grad_()
    w1 = dev_bf16(c["w1"]).requires_grad_()
    w2 = dev_bf16(c["w2"]).requires_grad_()
    p = dev_f32(c["probs"]).requires_grad_()
    y = gpu_lib.GroupedMLP.apply(x, p, w1, w2, list(k["split"]))
    y.backward(dev_bf16(c["dy"]))
    torch.cuda.synchronize()
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    want = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"], c["dy"], fwd)
    assert rel_norm(to_np(y.detach()), fwd["y"]) <= TOL
    assert rel_norm(to_np(x.grad), want["dx"]) <= TOL
    assert rel_norm(to_np(p.grad), want["dprobs"]) <= TOL
    assert rel_norm(to_np(w1.grad.float()), want["dw1"]) <= TOL


@pytest.mark.parametrize("name", ["ragged4", "many_small"])
def test_cached_weights_match_uncast_path(gpu_lib, name):
    """grouped_mlp_fwd_cached / grouped_mlp_bwd_cached on weights cast once by
    grouped_mlp_quantize_weights give bit-identical outputs to the calls that
    cast the bf16 weights themselves (same codes, same kernels), in training
    and inference, and the cache survives a second step with another split."""
    mx = gpu_lib
    k = CASES[name]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    x, w1, w2, dy = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"]), dev_bf16(c["dy"])
    p = dev_f32(c["probs"])
    split = c["split_sizes"].tolist()
    cache = mx.grouped_mlp_quantize_weights(w1, w2)

    def same(a, b):
        if a.dtype == torch.bfloat16:
            return torch.equal(a.view(torch.int16), b.view(torch.int16))
        return torch.equal(a.view(torch.int32), b.view(torch.int32))

    for split_now in (split, split[::-1]):
        y_ref, st_ref = mx.grouped_mlp_fwd(x, p, w1, w2, split_now, training=True)
        y_c, st_c = mx.grouped_mlp_fwd_cached(x, p, cache, split_now, training=True)
        y_i, _ = mx.grouped_mlp_fwd_cached(x, p, cache, split_now, training=False)
        ref = mx.grouped_mlp_bwd(dy, p, st_ref)
        got = mx.grouped_mlp_bwd_cached(dy, p, st_c, cache)
        torch.cuda.synchronize()
        assert same(y_ref, y_c) and same(y_ref, y_i)
        for a, b, what in zip(ref, got, ("dx", "dprobs", "dw1", "dw2")):
            assert same(a, b), what
    # and the cached path against the oracle directly
    want = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], c["split_sizes"])
    y_c, _ = mx.grouped_mlp_fwd_cached(x, p, cache, split, training=False)
    torch.cuda.synchronize()
    _check_rows(to_np(y_c), want["y"], split, "y (cached weights)")


def test_backward_on_user_stream_orders_side_work(gpu_lib):
    """grouped_mlp_bwd runs its wgrad GEMMs on a library side stream forked
    from and joined back into the caller's stream. Two accumulating calls on
    a user stream must give exactly twice one call's dW (fp32 doubling is
    exact): the second call's read-modify-write may start only after the
    first's, and everything is complete once the user stream is synchronized."""
    mx = gpu_lib
    k = CASES["two_tiles_ffn"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    x, w1, w2, dy = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"]), dev_bf16(c["dy"])
    p = dev_f32(c["probs"])
    split = c["split_sizes"].tolist()
    E, H, F = k["E"], k["H"], k["F"]
    user = torch.cuda.Stream()
    with torch.cuda.stream(user):
        _, st = mx.grouped_mlp_fwd(x, p, w1, w2, split, training=True, stream=user)
        once = [torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda"),
                torch.zeros((E, H, F), dtype=torch.float32, device="cuda")]
        twice = [torch.zeros_like(once[0]), torch.zeros_like(once[1])]
        dx1, dp1, _, _ = mx.grouped_mlp_bwd(dy, p, st, dw1=once[0], dw2=once[1], accumulate=True, stream=user)
        for _ in range(2):
            mx.grouped_mlp_bwd(dy, p, st, dw1=twice[0], dw2=twice[1], accumulate=True, stream=user)
    user.synchronize()
    for a, b in zip(twice, once):
        assert torch.equal(a, 2 * b)
    assert float(once[0].abs().sum()) > 0 and float(once[1].abs().sum()) > 0

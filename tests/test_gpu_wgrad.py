"""The fused backward's weight-gradient GEMMs (group-K, fp32 main grads)
against the oracle's float64 product of the very codes they multiply:
dW2_e = colwise(dY_e) . colwise(A_e)^T and dW1_e = colwise(dH1_e) .
colwise(X_e)^T over expert e's padded rows ("Efficient MoE training for
biological foundation models", Key technical approaches items 1 and 3; the
fp32 accumulation into main grads of "examples/llama: default-on fusion &
DP-comm perf toggles", Changes).

The columnwise dY and X copies come from the plain casts, which are
bit-exact against the oracle's quantize_colwise (the quantize tests), so the
oracle quantizes them itself; A and dH1 are requantized inside the fused
epilogues, so their codes and scales are read back from the call's buffers
(grouped_mlp_intermediates).

Bars: overwrite (accumulate=False) -- every element of the sampled rows of
dW within the MFMA's own error bound (tests.gpu_util.mfma_gemm_bound) of the
float64 product, an empty expert all zeros; accumulate -- from a random fp32
start I, every element equal to fl32(I + the overwrite result), bit for bit
(the epilogue adds the fp32 product to the old value once, round to nearest
even), an empty expert unchanged. The experts cover k ranges with a partial
last 128-column step, one shorter than a step, and an empty one."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, mfma_gemm_bound
from tests.test_gpu_intermediates import _bytes, _untile_colwise

pytestmark = pytest.mark.gpu

CASES = {
    # the tiny MoE workload (256 tokens, top-2 of 4, H=256, F=512, one empty expert)
    "tiny_moe": None,
    # padded k ranges 704 (5.5 steps), 0, 1120 (8.75 steps), 256 (2 steps);
    # dW1 is [4, 2048, 4096], 16 x 32 tiles per expert
    "moe_h4096_f1024": dict(seed=41, E=4, H=4096, F=1024, split=(700, 0, 1100, 248)),
    # k ranges of 64 (one partial step) and 160, more tiles along m than n
    "short_k": dict(seed=43, E=3, H=256, F=640, split=(40, 0, 129)),
}
SAMPLE_ROWS = 256    # rows of dW checked against the float64 product, per expert


def _inputs(name):
    if CASES[name] is None:
        return wl.make_mlp_inputs(wl.WORKLOADS["tiny_moe_fwd"], with_dy=True)
    c = CASES[name]
    return wl.small_mlp_case(c["seed"], c["E"], c["H"], c["F"], c["split"])


def _sample(rng, n):
    """Rows of a dW with n rows: all of them when few, else the first and last
    128-row tile and random rows in between."""
    if n <= SAMPLE_ROWS:
        return np.arange(n)
    ends = np.concatenate([np.arange(128), np.arange(n - 64, n)])
    mid = rng.choice(np.arange(128, n - 64), SAMPLE_ROWS - len(ends), replace=False)
    return np.sort(np.concatenate([ends, mid]))


@pytest.mark.parametrize("name", list(CASES))
def test_wgrad_on_its_own_operands(gpu_lib, name):
    c = _inputs(name)
    split = [int(s) for s in c["split_sizes"]]
    E, F2, H = c["w1"].shape
    F = F2 // 2
    R = sum(split)
    print(f"[wgrad] {name}: E={E} R={R} H={H} F={F} split={split}", flush=True)
    runner = gpu_lib.MLPRunner(E, R, H, F, split)
    probs = dev_f32(c["probs"])
    runner.forward(dev_bf16(c["x"]), probs, dev_bf16(c["w1"]), dev_bf16(c["w2"]), training=True)
    dw1 = torch.full((E, 2 * F, H), 5.0, dtype=torch.float32, device="cuda")
    dw2 = torch.full((E, H, F), 5.0, dtype=torch.float32, device="cuda")
    runner.backward(dev_bf16(c["dy"]), probs, dw1, dw2, accumulate=False)
    torch.cuda.synchronize()
    d1, d2 = dw1.cpu().numpy(), dw2.cpu().numpy()

    o = gpu_lib.mlp_intermediates(E, R, H, F, split)
    P = [(m + 31) // 32 * 32 for m in split]
    sumP, nq = sum(P), o["nq_col"]
    ac = orc.dequantize_rowwise(
        _bytes(runner.saved, o["a_col_codes"], F * sumP).reshape(F, sumP),
        _untile_colwise(_bytes(runner.saved, o["a_col_scales"], F // 32 * nq * 128), F, split, nq))
    dhc = orc.dequantize_rowwise(
        _bytes(runner.bwd_ws, o["dh1_col_codes"], 2 * F * sumP).reshape(2 * F, sumP),
        _untile_colwise(_bytes(runner.bwd_ws, o["dh1_col_scales"], 2 * F // 32 * nq * 128), 2 * F, split, nq))
    dyc = orc.dequantize_rowwise(*orc.quantize_colwise(orc.bf16_bits_to_f64(c["dy"]), split))
    xc = orc.dequantize_rowwise(*orc.quantize_colwise(orc.bf16_bits_to_f64(c["x"]), split))

    rng = np.random.default_rng(5)
    p0 = 0
    for e in range(E):
        ks = slice(p0, p0 + P[e])
        p0 += P[e]
        if split[e] == 0:
            assert not d1[e].any() and not d2[e].any(), f"empty expert {e}: dW not zero"
            continue
        for tag, got, lhs, rhs in (("dW2", d2[e], dyc, ac), ("dW1", d1[e], dhc, xc)):
            rows = _sample(rng, got.shape[0])
            A, B = lhs[rows, ks], rhs[:, ks]
            want = A @ B.T
            bound = mfma_gemm_bound(A, B)
            err = np.abs(got[rows].astype(np.float64) - want)
            worst = float(np.max(err / np.maximum(bound, 1e-300)))
            print(f"[wgrad] {name} {tag} expert {e}: k={P[e]}, {len(rows)} rows, worst error / MFMA bound "
                  f"{worst:.3f}", flush=True)
            assert np.all(err <= bound), f"{tag} expert {e}: error {worst:.2f}x the MFMA bound"

    # accumulate: one fp32 add of the same product into a random start
    i1 = rng.standard_normal((E, 2 * F, H)).astype(np.float32)
    i2 = rng.standard_normal((E, H, F)).astype(np.float32)
    a1, a2 = torch.from_numpy(i1).cuda(), torch.from_numpy(i2).cuda()
    runner.backward(dev_bf16(c["dy"]), probs, a1, a2, accumulate=True)
    torch.cuda.synchronize()
    for tag, got, start, prod in (("dW1", a1, i1, d1), ("dW2", a2, i2, d2)):
        want = start + prod                              # float32 + float32, round to nearest even
        same = got.cpu().numpy().view(np.uint32) == want.view(np.uint32)
        print(f"[wgrad] {name} {tag} accumulate: {int((~same).sum())} of {same.size} elements differ", flush=True)
        assert same.all(), f"{tag}: accumulated result is not fl32(start + product)"

"""GPU parity of the MXFP4 grouped MLP (grouped_mlp_fwd_fp4 /
grouped_mlp_bwd_fp4) against the oracle's MLP at quantize="mxfp4" (reading
R17: the MXFP8 MLP of "Efficient MoE training for biological foundation
models", Key technical approaches item 3, with every GEMM on MXFP4 copies).

Bar: as for the MXFP8 MLP, normwise relative error <= 2e-2 for Y, dX, dW1,
dW2 and dprobs, over the whole output and per expert with rows. One case is
shaped so that GEMM2 and dgrad1 run with a split-K tail. The GPU forms
A and dH1 in fp32 and the oracle in float64, so a requantized code can differ
by one E2M1 step where the two straddle a rounding boundary; such flips are
rare, and the measured errors are printed. An expert with no rows gets zero
dW (overwrite) or keeps its dW (accumulate)."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, rel_norm, to_np

pytestmark = pytest.mark.gpu
TOL = 2e-2

CASES = {
    "ragged4": dict(seed=130, E=4, H=256, F=384, split=(300, 0, 17, 200)),
    "two_tiles_ffn": dict(seed=131, E=3, H=512, F=768, split=(257, 33, 190)),
    "dense_one_expert": dict(seed=132, E=1, H=256, F=512, split=(384,)),
    "many_small": dict(seed=134, E=12, H=128, F=256,
                       split=(1, 31, 32, 33, 0, 64, 95, 96, 97, 127, 128, 129)),
    # 3 output tiles of GEMM2 and dgrad1 (n = H = 256): the whole launch is a
    # partial last round, so GEMM2 (k = 2048) runs split-K in 2 parts and
    # dgrad1 (k = 4096) in 4, partials summed by the reduce kernel
    "split_k_tail": dict(seed=135, E=2, H=256, F=2048, split=(300, 200)),
}


def _rows(got, want, split, what):
    err = rel_norm(got, want)
    print(f"  {what}: normwise {err:.2e}", flush=True)
    assert err <= TOL, what
    r0 = 0
    for e, m in enumerate(split):
        if m:
            ee = rel_norm(got[r0:r0 + m], want[r0:r0 + m])
            assert ee <= TOL, f"{what} expert {e}: {ee}"
        r0 += m


def _experts(got, want, split, what):
    err = rel_norm(got, want)
    print(f"  {what}: normwise {err:.2e}", flush=True)
    assert err <= TOL, what
    for e, m in enumerate(split):
        if m:
            ee = rel_norm(got[e], want[e])
            assert ee <= TOL, f"{what} expert {e}: {ee}"


def _fwd(mx, c, training):
    p = dev_f32(c["probs"])
    y, st = mx.grouped_mlp_fwd_fp4(dev_bf16(c["x"]), p, dev_bf16(c["w1"]), dev_bf16(c["w2"]),
                                   c["split_sizes"].tolist(), training=training)
    torch.cuda.synchronize()
    return y, st, p


@pytest.mark.parametrize("name", list(CASES))
def test_fp4_mlp_forward_backward(gpu_lib, name):
    k = CASES[name]
    print(f"[mlp_fp4] {name}: E={k['E']} H={k['H']} F={k['F']} split={k['split']}", flush=True)
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    split = list(k["split"])
    y, st, p = _fwd(gpu_lib, c, training=True)
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split, quantize="mxfp4")
    _rows(to_np(y), fwd["y"], split, "y")
    E, H, F = k["E"], k["H"], k["F"]
    dw1 = torch.full((E, 2 * F, H), 5.0, dtype=torch.float32, device="cuda")   # overwritten
    dw2 = torch.full((E, H, F), 5.0, dtype=torch.float32, device="cuda")
    dx, dp, dw1, dw2 = gpu_lib.grouped_mlp_bwd_fp4(dev_bf16(c["dy"]), p, st, dw1=dw1, dw2=dw2, accumulate=False)
    torch.cuda.synchronize()
    bwd = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], fwd, quantize="mxfp4")
    _rows(to_np(dx), bwd["dx"], split, "dx")
    _rows(to_np(dp)[:, None], bwd["dprobs"][:, None], split, "dprobs")
    _experts(to_np(dw1), bwd["dw1"], split, "dw1")
    _experts(to_np(dw2), bwd["dw2"], split, "dw2")
    for e, m in enumerate(split):
        if m == 0:
            assert torch.all(dw1[e] == 0) and torch.all(dw2[e] == 0), f"empty expert {e}"


def test_fp4_mlp_inference_matches_training(gpu_lib):
    k = CASES["ragged4"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    y1, st1, _ = _fwd(gpu_lib, c, training=False)
    y2, st2, _ = _fwd(gpu_lib, c, training=True)
    assert st1 is None and st2 is not None
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_fp4_mlp_accumulate_and_no_probs(gpu_lib):
    """accumulate=True adds into the fp32 main gradients (an empty expert keeps
    its values); probs None means routing weights 1."""
    k = CASES["ragged4"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"], probs="one")
    split = list(k["split"])
    E, H, F = k["E"], k["H"], k["F"]
    y, st = gpu_lib.grouped_mlp_fwd_fp4(dev_bf16(c["x"]), None, dev_bf16(c["w1"]), dev_bf16(c["w2"]), split)
    rng = np.random.default_rng(7)
    i1 = rng.standard_normal((E, 2 * F, H)).astype(np.float32) * 1e-3
    i2 = rng.standard_normal((E, H, F)).astype(np.float32) * 1e-3
    dw1, dw2 = torch.from_numpy(i1).cuda(), torch.from_numpy(i2).cuda()
    _, dp, dw1, dw2 = gpu_lib.grouped_mlp_bwd_fp4(dev_bf16(c["dy"]), None, st, dw1=dw1, dw2=dw2, accumulate=True)
    torch.cuda.synchronize()
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split, quantize="mxfp4")
    bwd = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], fwd, quantize="mxfp4",
                           dw1_in=i1, dw2_in=i2)
    _rows(to_np(y), fwd["y"], split, "y")
    _experts(to_np(dw1) - i1, bwd["dw1"] - i1, split, "dw1 increment")
    _experts(to_np(dw2) - i2, bwd["dw2"] - i2, split, "dw2 increment")
    assert np.array_equal(to_np(dw1)[1], i1[1]) and np.array_equal(to_np(dw2)[1], i2[1]), "empty expert changed"


def test_fp4_mlp_differs_from_mxfp8(gpu_lib):
    """The MXFP4 forward is not the MXFP8 one: on the same inputs the two
    outputs differ by about the MXFP4 quantization error, and each matches its
    own oracle."""
    k = CASES["ragged4"]
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    split = list(k["split"])
    y4, _, _ = _fwd(gpu_lib, c, training=False)
    y8, _ = gpu_lib.grouped_mlp_fwd(dev_bf16(c["x"]), dev_f32(c["probs"]), dev_bf16(c["w1"]), dev_bf16(c["w2"]),
                                    split, training=False)
    torch.cuda.synchronize()
    w4 = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split, quantize="mxfp4")["y"]
    w8 = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split)["y"]
    gap = rel_norm(w4, w8)
    assert gap > 5 * TOL                      # the formats really differ on these inputs
    assert rel_norm(to_np(y4), w4) <= TOL and rel_norm(to_np(y8), w8) <= TOL


@pytest.mark.parametrize("name", ["ragged4", "split_k_tail"])
def test_fp4_cached_weights_match_uncast_path(gpu_lib, name):
    """grouped_mlp_fwd_fp4_cached / grouped_mlp_bwd_fp4_cached on weights cast
    once by grouped_mlp_fp4_quantize_weights give bit-identical outputs to the
    calls that cast the bf16 weights themselves (same codes, same kernels), in
    training and inference, overwriting and accumulating the weight gradients,
    and the cache serves a second step with another split; the cached path
    also meets the oracle's bar on its own."""
    mx = gpu_lib
    k = CASES[name]
    print(f"[mlp_fp4 cached] {name}: E={k['E']} H={k['H']} F={k['F']} split={k['split']}", flush=True)
    c = wl.small_mlp_case(k["seed"], k["E"], k["H"], k["F"], k["split"])
    x, w1, w2, dy = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"]), dev_bf16(c["dy"])
    p = dev_f32(c["probs"])
    split = list(k["split"])
    E, H, F = k["E"], k["H"], k["F"]
    cache = mx.grouped_mlp_fp4_quantize_weights(w1, w2)

    def same(a, b):
        if a.dtype == torch.bfloat16:
            return torch.equal(a.view(torch.int16), b.view(torch.int16))
        return torch.equal(a.view(torch.int32), b.view(torch.int32))

    rng = np.random.default_rng(11)
    start1 = torch.from_numpy(rng.standard_normal((E, 2 * F, H)).astype(np.float32) * 1e-3).cuda()
    start2 = torch.from_numpy(rng.standard_normal((E, H, F)).astype(np.float32) * 1e-3).cuda()
    for split_now in (split, split[::-1]):
        y_ref, st_ref = mx.grouped_mlp_fwd_fp4(x, p, w1, w2, split_now, training=True)
        y_c, st_c = mx.grouped_mlp_fwd_fp4_cached(x, p, cache, split_now, training=True)
        y_i, _ = mx.grouped_mlp_fwd_fp4_cached(x, p, cache, split_now, training=False)
        ref = mx.grouped_mlp_bwd_fp4(dy, p, st_ref)
        got = mx.grouped_mlp_bwd_fp4_cached(dy, p, st_c, cache)
        acc_ref = mx.grouped_mlp_bwd_fp4(dy, p, st_ref, dw1=start1.clone(), dw2=start2.clone(), accumulate=True)
        acc_got = mx.grouped_mlp_bwd_fp4_cached(dy, p, st_c, cache, dw1=start1.clone(), dw2=start2.clone(),
                                                accumulate=True)
        torch.cuda.synchronize()
        assert same(y_ref, y_c) and same(y_ref, y_i), "y"
        for a, b, what in zip(ref + acc_ref, got + acc_got,
                              ("dx", "dprobs", "dw1", "dw2", "dx (acc)", "dprobs (acc)", "dw1 (acc)", "dw2 (acc)")):
            assert same(a, b), what
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split, quantize="mxfp4")
    y_c, st_c = mx.grouped_mlp_fwd_fp4_cached(x, p, cache, split, training=True)
    dx, dp, dw1, dw2 = mx.grouped_mlp_bwd_fp4_cached(dy, p, st_c, cache)
    torch.cuda.synchronize()
    bwd = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], fwd, quantize="mxfp4")
    _rows(to_np(y_c), fwd["y"], split, "y (cached weights)")
    _rows(to_np(dx), bwd["dx"], split, "dx (cached weights)")
    _experts(to_np(dw1), bwd["dw1"], split, "dw1 (cached weights)")
    _experts(to_np(dw2), bwd["dw2"], split, "dw2 (cached weights)")


def test_fp4_cached_weights_bit_identical_fullsize(gpu_lib):
    """The Mixtral-shaped MXFP4 forward + backward (accumulating into fp32
    main grads) on weights cast once into the MXFP4 weight cache equals the
    step that casts the bf16 weights itself, bit for bit, at full size: the
    cache's per-expert columnwise copies feed dgrad2 and dgrad1 at their
    real offsets and extents."""
    mx = gpu_lib
    w = wl.WORKLOADS["mixtral_moe_fwd_bwd"]
    print("[mlp_fp4 cached] mixtral_moe_fwd_bwd: generating inputs", flush=True)
    c = wl.make_mlp_inputs(w, with_dy=True)
    split = c["split_sizes"].tolist()
    E, H, F = w.experts, w.hidden, w.ffn
    x, w1, w2, dy = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"]), dev_bf16(c["dy"])
    p = dev_f32(c["probs"])
    same = lambda a, b: torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                                    b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))
    print("[mlp_fp4 cached] reference step", flush=True)
    y_ref, st = mx.grouped_mlp_fwd_fp4(x, p, w1, w2, split, training=True)
    ref = mx.grouped_mlp_bwd_fp4(dy, p, st, dw1=torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda"),
                                 dw2=torch.zeros((E, H, F), dtype=torch.float32, device="cuda"), accumulate=True)
    del st
    print("[mlp_fp4 cached] cached step", flush=True)
    cache = mx.grouped_mlp_fp4_quantize_weights(w1, w2)
    y, st = mx.grouped_mlp_fwd_fp4_cached(x, p, cache, split, training=True)
    got = mx.grouped_mlp_bwd_fp4_cached(dy, p, st, cache,
                                        dw1=torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda"),
                                        dw2=torch.zeros((E, H, F), dtype=torch.float32, device="cuda"),
                                        accumulate=True)
    torch.cuda.synchronize()
    assert same(y, y_ref), "y"
    for a, b, what in zip(got, ref, ("dx", "dprobs", "dw1", "dw2")):
        assert same(a, b), what


def test_fp4_mlp_fullsize_sampled(gpu_lib):
    """The Mixtral-8x7B-shaped MoE MLP forward + backward at MXFP4 (4096
    tokens top-2 of 8: 8192 rows, H = 4096, F = 14336), in the calls the
    benchmark times (training forward, backward accumulating into zeroed fp32
    gradients), on the rows and dW entries whose expected values
    tests/golden/make_fullsize.py --mxfp4 computed from the oracle alone."""
    import os
    from tests.golden.make_fullsize import golden_path
    name = "mixtral_moe_fwd_bwd"
    path = golden_path(name, "mxfp4")
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not generated")
    g = np.load(path, allow_pickle=False)
    w = wl.WORKLOADS[name]
    print(f"[mlp_fp4 fullsize] {name}: generating inputs", flush=True)
    c = wl.make_mlp_inputs(w, with_dy=True)
    split = c["split_sizes"].astype(np.int64)
    assert np.array_equal(split, g["split"]), "input generator drifted from the stored sample"
    E, H, F = w.experts, w.hidden, w.ffn
    p = dev_f32(c["probs"])
    print(f"[mlp_fp4 fullsize] {name}: forward", flush=True)
    y, st = gpu_lib.grouped_mlp_fwd_fp4(dev_bf16(c["x"]), p, dev_bf16(c["w1"]), dev_bf16(c["w2"]), split.tolist())
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda")
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device="cuda")
    print(f"[mlp_fp4 fullsize] {name}: backward", flush=True)
    dx, dp, dw1, dw2 = gpu_lib.grouped_mlp_bwd_fp4(dev_bf16(c["dy"]), p, st, dw1=dw1, dw2=dw2, accumulate=True)
    torch.cuda.synchronize()
    sel = torch.from_numpy(g["rows"]).cuda()
    for key, t in (("y", y), ("dx", dx)):
        got = to_np(t[sel])
        errs = [rel_norm(got[i], g[key][i]) for i in range(len(g["rows"]))]
        print(f"[mlp_fp4 fullsize] {key} max row error {max(errs):.2e}", flush=True)
        assert max(errs) <= TOL, key
    err = rel_norm(to_np(dp[sel]), g["dprobs"])
    print(f"[mlp_fp4 fullsize] dprobs error {err:.2e}", flush=True)
    assert err <= TOL
    for key, buf in (("dw1", dw1), ("dw2", dw2)):
        idx = g[f"{key}_idx"]
        got = buf[tuple(torch.from_numpy(idx[:, k]).cuda() for k in range(3))].cpu().numpy().astype(np.float64)
        for e in np.unique(idx[:, 0]).tolist():
            m = idx[:, 0] == e
            err = rel_norm(got[m], g[key][m])
            print(f"[mlp_fp4 fullsize] {key} expert {e} error {err:.2e}", flush=True)
            assert err <= TOL, f"{key} expert {e}: {err}"

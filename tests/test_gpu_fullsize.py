"""GPU parity at full size, in the launch configuration the benchmark times
(MLPRunner: training forward, then backward accumulating into fp32 weight
gradients), on sampled outputs whose expected values the oracle computed one
by one (tests/golden/make_fullsize.py writes them; the inputs are regenerated
here from the workload seed).

Workloads: the Llama-3.1-8B dense MLP forward (8192 x 4096 -> 14336), the
Mixtral-8x7B-shaped MoE forward (8192 tokens, top-2 of 8) and the MoE
forward + backward (4096 tokens) ("Efficient MoE training for biological
foundation models", Key technical approaches; TE Llama 3 recipe, MXFP8 vs
BF16 throughput table).

Bar: normwise relative error <= 2e-2 per sampled row (Y, dX), over the
sampled dprobs, and over each expert's sampled dW1 / dW2 entries - the same
bar as the small-size MLP tests, for the same reason (requantized
intermediates may sit one code apart where fp32 and fp64 straddle a rounding
boundary)."""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from tests.golden.make_fullsize import FULLSIZE, golden_path
from tests.gpu_util import dev_bf16, dev_f32, rel_norm, to_np

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.mark.parametrize("name", FULLSIZE)
def test_fullsize_sampled(gpu_lib, name):
    path = golden_path(name)
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not generated")
    g = np.load(path, allow_pickle=False)
    w = wl.WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    c = wl.make_mlp_inputs(w, with_dy=w.backward)
    split = c["split_sizes"].astype(np.int64)
    assert np.array_equal(split, g["split"]), "input generator drifted from the stored sample"
    E, R, H, F = w.experts, w.rows, w.hidden, w.ffn

    x, w1, w2 = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"])
    probs = dev_f32(c["probs"])
    runner = gpu_lib.MLPRunner(E, R, H, F, split.tolist())
    print(f"[fullsize] {name}: forward", flush=True)
    y = runner.forward(x, probs, w1, w2, training=w.backward)
    torch.cuda.synchronize()
    rows = g["rows"]
    y_rows = to_np(y[torch.from_numpy(rows).cuda()])
    errs = [rel_norm(y_rows[i], g["y"][i]) for i in range(len(rows))]
    print(f"[fullsize] {name}: y max row error {max(errs):.2e}", flush=True)
    for r, err in zip(rows.tolist(), errs):
        assert err <= TOL, f"y row {r}: {err}"
    if not w.backward:
        return

    dy = dev_bf16(c["dy"])
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda")
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device="cuda")
    print(f"[fullsize] {name}: backward", flush=True)
    dx, dprobs = runner.backward(dy, probs, dw1, dw2, accumulate=True)
    torch.cuda.synchronize()
    sel = torch.from_numpy(rows).cuda()
    dx_rows = to_np(dx[sel])
    errs = [rel_norm(dx_rows[i], g["dx"][i]) for i in range(len(rows))]
    dp_err = rel_norm(to_np(dprobs[sel]), g["dprobs"])
    print(f"[fullsize] {name}: dx max row error {max(errs):.2e}, dprobs {dp_err:.2e}", flush=True)
    for r, err in zip(rows.tolist(), errs):
        assert err <= TOL, f"dx row {r}: {err}"
    assert dp_err <= TOL, "dprobs"
    for key, buf in (("dw1", dw1), ("dw2", dw2)):
        idx = g[f"{key}_idx"]
        got = buf[tuple(torch.from_numpy(idx[:, k]).cuda() for k in range(3))].cpu().numpy().astype(np.float64)
        for e in np.unique(idx[:, 0]).tolist():
            m = idx[:, 0] == e
            err = rel_norm(got[m], g[key][m])
            print(f"[fullsize] {name}: {key} expert {e} error {err:.2e}", flush=True)
            assert err <= TOL, f"{key} expert {e}: {err}"


def test_fullsize_cached_weights_bit_identical(gpu_lib):
    """The Mixtral-shaped forward + backward on weights cast once into the
    weight cache (grouped_mlp_quantize_weights, then the *_cached calls)
    equals the step that casts the bf16 weights itself, bit for bit, at full
    size. At this shape the cache is a whole number of 2 MiB pages, so the
    dgrad GEMMs' loads of the columnwise weight scales must stay inside it."""
    name = "mixtral_moe_fwd_bwd"
    w = wl.WORKLOADS[name]
    print(f"[fullsize] {name} cached weights: generating inputs", flush=True)
    c = wl.make_mlp_inputs(w, with_dy=True)
    split = c["split_sizes"].tolist()
    E, R, H, F = w.experts, w.rows, w.hidden, w.ffn
    x, w1, w2, dy = dev_bf16(c["x"]), dev_bf16(c["w1"]), dev_bf16(c["w2"]), dev_bf16(c["dy"])
    probs = dev_f32(c["probs"])
    runner = gpu_lib.MLPRunner(E, R, H, F, split)
    grads = [torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda"),
             torch.zeros((E, H, F), dtype=torch.float32, device="cuda")]
    print(f"[fullsize] {name} cached weights: reference step", flush=True)
    y_ref = runner.forward(x, probs, w1, w2, training=True).clone()
    dx_ref, dp_ref = (t.clone() for t in runner.backward(dy, probs, *grads, accumulate=True))
    cache_bytes = gpu_lib.grouped_mlp_weight_cache_bytes(E, H, F)
    assert cache_bytes % (2 << 20) == 0
    runner.quantize_weights(w1, w2)
    grads_c = [torch.zeros_like(grads[0]), torch.zeros_like(grads[1])]
    print(f"[fullsize] {name} cached weights: cached step", flush=True)
    y = runner.forward_cached(x, probs, training=True)
    dx, dp = runner.backward_cached(dy, probs, *grads_c, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16))
    assert torch.equal(dp.view(torch.int32), dp_ref.view(torch.int32))
    for a, b in zip(grads_c, grads):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    print(f"[fullsize] {name} cached weights: bit-identical", flush=True)

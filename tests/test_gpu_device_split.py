"""GPU parity of the fused MLP with device-resident split sizes
(grouped_mlp_fwd_device_split / grouped_mlp_bwd_device_split): the
per-expert row counts GroupedLinear takes ("Efficient MoE training for
biological foundation models", Key technical approaches item 1) stay in
device memory and the call's first kernel builds every group table from
them.

Expected values: the host-split calls (grouped_mlp_fwd / _bwd and their
gather forms, themselves checked against the oracle in test_gpu_mlp.py and
test_gpu_moe.py) on the same inputs and the same (clamped) split, restricted
to the routed rows. Where the host-split call uses no split-K tail (ffn <= 384
here: fewer than 8 k-steps in GEMM2 and dgrad1), both run the same tiles over
the same k ranges, so every output must be bit-identical. With a split-K tail
in the host call (ffn = 1024), y and dX may differ in the fp32 summation order
of the tail tiles; there the bar is the oracle's 2e-2 normwise plus 4e-3
normwise against the host call (one bf16 rounding). Rows past the routed ones
must keep their previous contents in y and dX, and dprobs must be 0 there.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, rel_norm, to_np

pytestmark = pytest.mark.gpu
PATTERN = -7.0                         # prior contents of y / dx rows past the routed ones


def _case(seed, E, H, F, split, extra_rows):
    """Inputs for E experts with `split`, plus extra_rows unrouted rows at the
    end of x / dy / probs (generated as a ghost expert, then dropped)."""
    c = wl.small_mlp_case(seed, E + 1, H, F, tuple(split) + (extra_rows,))
    c["w1"], c["w2"] = c["w1"][:E], c["w2"][:E]
    return c


def _host_run(mx, c, split, S):
    E, F2, H = c["w1"].shape
    F = F2 // 2
    run = mx.MLPRunner(E, S, H, F, split)
    x = dev_bf16(c["x"][:S])
    p = dev_f32(c["probs"][:S])
    run.forward(x, p, dev_bf16(c["w1"]), dev_bf16(c["w2"]), training=True)
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda")
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device="cuda")
    run.backward(dev_bf16(c["dy"][:S]), p, dw1, dw2, accumulate=False)
    torch.cuda.synchronize()
    return dict(y=run.y.clone(), dx=run.dx.clone(), dprobs=run.dprobs.clone(), dw1=dw1, dw2=dw2)


def _dev_run(mx, c, counts, R):
    E, F2, H = c["w1"].shape
    F = F2 // 2
    run = mx.DeviceSplitMLPRunner(E, R, H, F)
    run.y.fill_(PATTERN)
    run.dx.fill_(PATTERN)
    run.dprobs.fill_(PATTERN)
    cnt = torch.tensor(counts, dtype=torch.int64, device="cuda")
    p = dev_f32(c["probs"])
    run.forward(cnt, dev_bf16(c["x"]), p, dev_bf16(c["w1"]), dev_bf16(c["w2"]), training=True)
    # non-zero prior contents: experts with no rows must be zeroed (accumulate off)
    dw1 = torch.full((E, 2 * F, H), 3.0, dtype=torch.float32, device="cuda")
    dw2 = torch.full((E, H, F), 3.0, dtype=torch.float32, device="cuda")
    run.backward(cnt, dev_bf16(c["dy"]), p, dw1, dw2, accumulate=False)
    torch.cuda.synchronize()
    return dict(y=run.y, dx=run.dx, dprobs=run.dprobs, dw1=dw1, dw2=dw2)


def _same(a, b, what):
    assert a.shape == b.shape, what
    ai = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
    bi = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
    n = int((ai != bi).sum())
    assert n == 0, f"{what}: {n} of {a.numel()} elements differ"


def _check_tail(got, S):
    if S < got["y"].shape[0]:
        assert torch.all(got["y"][S:] == PATTERN), "y rows past the routed ones were written"
        assert torch.all(got["dx"][S:] == PATTERN), "dx rows past the routed ones were written"
        assert torch.all(got["dprobs"][S:] == 0), "dprobs past the routed rows is not 0"


def _clamp(counts, R):
    out, run = [], 0
    for c in counts:
        c = max(int(c), 0)
        c = min(c, R - run)
        out.append(c)
        run += c
    return out


CASES = {
    # (seed, E, H, F, counts, rows of x)
    "ragged": (50, 4, 256, 384, (300, 0, 17, 200), 517),
    "dropped_rows": (51, 4, 256, 256, (100, 0, 57, 3), 256),
    "many_small": (52, 12, 128, 256, (1, 31, 32, 33, 0, 64, 95, 96, 97, 127, 128, 129), 900),
    "one_expert": (53, 1, 256, 384, (384,), 384),
    # a negative count reads as 0; counts past R are cut at R
    "clamped": (54, 3, 256, 256, (-5, 300, 50), 320),
}


@pytest.mark.parametrize("name", list(CASES))
def test_device_split_matches_host_split(gpu_lib, name):
    seed, E, H, F, counts, R = CASES[name]
    split = _clamp(counts, R)
    S = sum(split)
    print(f"[device_split] {name}: E={E} R={R} H={H} F={F} counts={counts} -> {split}", flush=True)
    c = _case(seed, E, H, F, split, R - S)
    got = _dev_run(gpu_lib, c, counts, R)
    want = _host_run(gpu_lib, c, split, S)
    for k in ("y", "dx", "dprobs"):
        _same(got[k][:S], want[k], k)
    for k in ("dw1", "dw2"):
        _same(got[k], want[k], k)
    _check_tail(got, S)


def test_device_split_all_rows_dropped(gpu_lib):
    """Every count 0: nothing routed; y / dx untouched, dprobs 0, dW zeroed."""
    E, H, F, R = 3, 128, 128, 96
    c = _case(55, E, H, F, (0, 0, 0), R)
    got = _dev_run(gpu_lib, c, (0, 0, 0), R)
    _check_tail(got, 0)
    assert torch.all(got["dw1"] == 0) and torch.all(got["dw2"] == 0)


def test_device_split_with_split_k_tail_in_host_call(gpu_lib):
    """ffn = 1024: the host call splits GEMM2's and dgrad1's last tiles over
    k; the device-split call does not."""
    E, H, F = 2, 256, 1024
    split = [300, 100]
    c = _case(56, E, H, F, split, 64)
    got = _dev_run(gpu_lib, c, split, 464)
    want = _host_run(gpu_lib, c, split, 400)
    fwd = orc.mlp_forward(c["x"][:400], c["probs"][:400], c["w1"], c["w2"], split)
    bwd = orc.mlp_backward(c["x"][:400], c["probs"][:400], c["w1"], c["w2"], split, c["dy"][:400], fwd)
    for k, ref in (("y", fwd["y"]), ("dx", bwd["dx"])):
        e_host = rel_norm(to_np(got[k][:400]), to_np(want[k]))
        e_orc = rel_norm(to_np(got[k][:400]), ref)
        print(f"[device_split] split-K case {k}: vs host call {e_host:.2e}, vs oracle {e_orc:.2e}", flush=True)
        assert e_host <= 4e-3 and e_orc <= 2e-2, k
    for k in ("dprobs", "dw1", "dw2"):
        _same(got[k][:400] if k == "dprobs" else got[k], want[k], k)
    _check_tail(got, 400)


def test_device_split_cached_weights_bit_identical(gpu_lib):
    seed, E, H, F, counts, R = CASES["dropped_rows"]
    c = _case(seed, E, H, F, counts, R - sum(counts))
    got = _dev_run(gpu_lib, c, counts, R)
    run = gpu_lib.DeviceSplitMLPRunner(E, R, H, F)
    cache = gpu_lib.WeightCache(E, H, F)
    gpu_lib.grouped_mlp_quantize_weights(dev_bf16(c["w1"]), dev_bf16(c["w2"]), cache)
    cnt = torch.tensor(counts, dtype=torch.int64, device="cuda")
    p = dev_f32(c["probs"])
    run.forward(cnt, dev_bf16(c["x"]), p, cache=cache)
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda")
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device="cuda")
    run.backward(cnt, dev_bf16(c["dy"]), p, dw1, dw2, accumulate=False, cache=cache)
    torch.cuda.synchronize()
    S = sum(counts)
    _same(run.y[:S], got["y"][:S], "y")
    _same(run.dx[:S], got["dx"][:S], "dx")
    _same(dw1, got["dw1"], "dw1")
    _same(dw2, got["dw2"], "dw2")


def test_dispatch_counts_feed_the_mlp_without_a_host_copy(gpu_lib):
    """Token dispatch (with dropped entries) -> its device counts and
    row_token -> the device-split MLP with the gather fused into the casts,
    against the host-split gather calls on counts copied to the host."""
    T, k, E, H, F = 300, 2, 4, 256, 256
    rng = np.random.default_rng(57)
    x = dev_bf16(wl.normal_bf16(rng, (T, H), 1.0))
    dy = dev_bf16(wl.normal_bf16(rng, (T, H), 1e-3))
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[::7, 1] = E                                   # dropped entries
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w1 = dev_bf16(wl.normal_bf16(rng, (E, 2 * F, H), 0.02))
    w2 = dev_bf16(wl.normal_bf16(rng, (E, H, F), 0.02))
    R = T * k
    _, probs, _, row_token, counts = gpu_lib.mx_moe_dispatch(x, torch.from_numpy(idx).cuda(),
                                                             torch.from_numpy(w).cuda(), E, gather=False)
    run = gpu_lib.DeviceSplitMLPRunner(E, R, H, F)
    run.forward(counts, x, probs, w1, w2, row_token=row_token)
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda")
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device="cuda")
    run.backward(counts, dy, probs, dw1, dw2, accumulate=False, row_token=row_token)
    torch.cuda.synchronize()

    split = counts.cpu().tolist()
    S = sum(split)
    assert S == R - len(range(0, T, 7))
    y_h, st = gpu_lib.grouped_mlp_fwd_gather(x, row_token[:S].contiguous(), probs[:S].contiguous(), w1, w2, split)
    dx_h, dp_h, dw1_h, dw2_h = gpu_lib.grouped_mlp_bwd_gather(dy, row_token[:S].contiguous(),
                                                              probs[:S].contiguous(), st)
    torch.cuda.synchronize()
    _same(run.y[:S], y_h, "y")
    _same(run.dx[:S], dx_h, "dx")
    _same(run.dprobs[:S], dp_h, "dprobs")
    _same(dw1, dw1_h, "dw1")
    _same(dw2, dw2_h, "dw2")

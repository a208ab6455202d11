"""Parity of the intermediates that the fused epilogues requantize inside the
call, read back from the caller's buffers (grouped_mlp_intermediates gives
their offsets): A = w * silu(g) * u of the forward (rowwise for GEMM2, grouped
columnwise for wgrad2), dH1 = [dg | du] of the backward (rowwise for dgrad1,
grouped columnwise for wgrad1), and the saved bf16 H1.

These are the intermediates the fused GroupedLinear -> ScaledSwiGLU ->
GroupedLinear op and its backward keep out of HBM in 16/32-bit form
("Efficient MoE training for biological foundation models", Key technical
approaches item 3).

Expected values: the oracle's own float64 A and dH1 (mlp_forward /
mlp_backward on the same seeded inputs), quantized by the oracle. The GPU
forms A and dH1 in fp32 from fp32 accumulators, the oracle in float64, so a
code may sit one step away where the two values straddle a rounding
boundary, and a block scale may differ by one where the block amax straddles
a power of two. Bar: every differing code is exactly one E4M3 step apart
(same scale) or, in a block whose scale differs by one, within one step of
the coarser grid; the fraction of differing codes (counting every element of
a block whose scale differs) is at most 1e-3. The rates are printed.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, mfma_gemm_bound

pytestmark = pytest.mark.gpu
MAX_RATE = 1e-3

CASES = {
    # the tiny MoE workload (256 tokens, top-2 of 4, H=256, F=512, one empty expert)
    "tiny_moe": None,
    # GEMM1 and dgrad2 contract over H = 4096 as in the Llama / Mixtral shapes;
    # ragged experts, one empty, partial 32-row blocks
    "moe_h4096_f1024": dict(seed=41, E=4, H=4096, F=1024, split=(700, 0, 1100, 248)),
}


def _inputs(name):
    if CASES[name] is None:
        return wl.make_mlp_inputs(wl.WORKLOADS["tiny_moe_fwd"], with_dy=True)
    c = CASES[name]
    return wl.small_mlp_case(c["seed"], c["E"], c["H"], c["F"], c["split"])


def _bytes(buf, off, n):
    return buf[off:off + n].cpu().numpy()


def _untile_rowwise(raw, rows, K):
    """k-tiled scales of a rowwise [rows, K] code matrix -> row-major [rows, K/32]."""
    nq = K // 128
    r = np.arange(rows)[:, None]
    b = np.arange(K // 32)[None, :]
    return raw[((r >> 5) * nq + b // 4) * 128 + (r & 31) * 4 + b % 4]


def _untile_colwise(raw, cols, split, nq_col):
    """k-tiled scales of a grouped columnwise [cols, sumP] code matrix ->
    row-major [cols, sumP/32] (expert e's blocks start at step q0_e)."""
    P = [(m + 31) // 32 * 32 for m in split]
    out = np.zeros((cols, sum(P) // 32), np.uint8)
    c = np.arange(cols)[:, None]
    q0, b0 = 0, 0
    for p in P:
        bl = np.arange(p // 32)[None, :]
        out[:, b0:b0 + p // 32] = raw[((c >> 5) * nq_col + q0 + bl // 4) * 128 + (c & 31) * 4 + bl % 4]
        q0 += -(-p // 128)
        b0 += p // 32
    return out


def _grid_index(codes):
    """Signed position of an E4M3 code on the value grid (+-0 -> 0)."""
    c = codes.astype(np.int64)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


def _compare(tag, q_gpu, s_gpu, q_ref, s_ref):
    rows, cols = q_ref.shape
    assert q_gpu.shape == q_ref.shape and s_gpu.shape == s_ref.shape, tag
    ds = np.abs(s_gpu.astype(np.int64) - s_ref.astype(np.int64))
    assert ds.max() <= 1, f"{tag}: a block scale differs by {ds.max()}"
    same = ds == 0
    d = np.abs(_grid_index(q_gpu) - _grid_index(q_ref)).reshape(rows, cols // 32, 32)
    worst = int(d[same].max()) if same.any() else 0
    assert worst <= 1, f"{tag}: a code differs by {worst} steps under the same scale"
    code_mis = int((d[same] > 0).sum())
    # blocks whose scale differs by one: values within one step of the coarser grid
    if (~same).any():
        sc = np.maximum(s_gpu, s_ref).astype(np.float64)[~same]
        vg = (orc.e4m3_value(q_gpu).reshape(rows, cols // 32, 32) * orc.e8m0_value(s_gpu)[..., None])[~same]
        vo = (orc.e4m3_value(q_ref).reshape(rows, cols // 32, 32) * orc.e8m0_value(s_ref)[..., None])[~same]
        step = np.maximum(2.0 ** -3 * np.maximum(np.abs(vg), np.abs(vo)), 2.0 ** (sc[:, None] - 127 - 9))
        assert np.all(np.abs(vg - vo) <= step * (1 + 1e-12)), f"{tag}: a re-scaled block is off by more than a step"
    mis = code_mis + 32 * int((~same).sum())
    rate = mis / q_ref.size
    print(f"[intermediates] {tag}: {code_mis} codes one step apart, {int((~same).sum())} of {same.size} "
          f"block scales one apart; mismatch rate {rate:.2e} over {q_ref.size} codes", flush=True)
    assert rate <= MAX_RATE, f"{tag}: mismatch rate {rate}"
    return rate


@pytest.mark.parametrize("name", list(CASES))
def test_requantized_intermediates_match_oracle(gpu_lib, name):
    c = _inputs(name)
    split = [int(s) for s in c["split_sizes"]]
    E, F2, H = c["w1"].shape                      # W1 is [E, 2F, H]
    F = F2 // 2
    R = sum(split)
    print(f"[intermediates] {name}: E={E} R={R} H={H} F={F} split={split}", flush=True)
    runner = gpu_lib.MLPRunner(E, R, H, F, split)
    probs = dev_f32(c["probs"])
    runner.forward(dev_bf16(c["x"]), probs, dev_bf16(c["w1"]), dev_bf16(c["w2"]), training=True)
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device="cuda")
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device="cuda")
    runner.backward(dev_bf16(c["dy"]), probs, dw1, dw2, accumulate=True)
    torch.cuda.synchronize()
    o = gpu_lib.mlp_intermediates(E, R, H, F, split)
    P = sum((m + 31) // 32 * 32 for m in split)
    nq, R32 = o["nq_col"], -(-R // 32) * 32

    print(f"[intermediates] {name}: oracle forward + backward", flush=True)
    fwd = orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], split)
    bwd = orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], fwd)

    # saved H1 (bf16): within the GEMM's own error bound plus one bf16
    # rounding on each side (outputs that cancel to near zero keep the
    # GEMM's absolute error, so a relative bf16 bar alone does not hold)
    h1_bits = _bytes(runner.saved, o["h1"], R * 2 * F * 2).view(np.uint16).reshape(R, 2 * F)
    h1_gpu = orc.bf16_bits_to_f64(h1_bits)
    xh = orc.dequantize_rowwise(*orc.quantize_rowwise(orc.bf16_bits_to_f64(c["x"])))
    off = np.concatenate([[0], np.cumsum(split)])
    bound = np.zeros((R, 2 * F))
    for e in range(E):
        if split[e]:
            w1h = orc.dequantize_rowwise(*orc.quantize_rowwise(orc.bf16_bits_to_f64(c["w1"][e])))
            bound[off[e]:off[e + 1]] = mfma_gemm_bound(xh[off[e]:off[e + 1]], w1h)
    dh = np.abs(h1_gpu - fwd["h1_bf16"])
    lim = bound + 2.0 ** -8 * (np.abs(fwd["h1"]) + np.abs(h1_gpu))
    assert np.all(dh <= lim), f"H1 off by {float(np.max(dh / np.maximum(lim, 1e-300))):.2f}x the bound"
    print(f"[intermediates] {name}: H1 bf16 differs at a rate of {np.mean(dh > 0):.2e}", flush=True)

    # A: rowwise [R, F] and grouped columnwise [F, sumP]
    a_q = _bytes(runner.fwd_ws, o["a_row_codes"], R * F).reshape(R, F)
    a_s = _untile_rowwise(_bytes(runner.fwd_ws, o["a_row_scales"], R32 * F // 32), R, F)
    rq, rs = orc.quantize_rowwise(fwd["a"])
    _compare(f"{name} A rowwise", a_q, a_s, rq, rs)
    ac_q = _bytes(runner.saved, o["a_col_codes"], F * P).reshape(F, P)
    ac_s = _untile_colwise(_bytes(runner.saved, o["a_col_scales"], F // 32 * nq * 128), F, split, nq)
    cq, cs = orc.quantize_colwise(fwd["a"], split)
    _compare(f"{name} A columnwise", ac_q, ac_s, cq, cs)

    # dH1: rowwise [R, 2F] and grouped columnwise [2F, sumP]
    d_q = _bytes(runner.bwd_ws, o["dh1_row_codes"], R * 2 * F).reshape(R, 2 * F)
    d_s = _untile_rowwise(_bytes(runner.bwd_ws, o["dh1_row_scales"], R32 * 2 * F // 32), R, 2 * F)
    rq, rs = orc.quantize_rowwise(bwd["dh1"])
    _compare(f"{name} dH1 rowwise", d_q, d_s, rq, rs)
    dc_q = _bytes(runner.bwd_ws, o["dh1_col_codes"], 2 * F * P).reshape(2 * F, P)
    dc_s = _untile_colwise(_bytes(runner.bwd_ws, o["dh1_col_scales"], 2 * F // 32 * nq * 128), 2 * F, split, nq)
    cq, cs = orc.quantize_colwise(bwd["dh1"], split)
    _compare(f"{name} dH1 columnwise", dc_q, dc_s, cq, cs)

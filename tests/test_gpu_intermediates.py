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
forms A and dH1 in fp32 from its fp32 GEMM outputs, the oracle in float64, so
the two values differ by the GEMM's error carried through the epilogue's
arithmetic (largest, relative to the block, for elements that cancel towards
zero, where the E4M3 grid is finest) and may then round to different codes,
and a block scale may differ by one where the block amax straddles a power of
two. Bars: every dequantized value within that carried error (the MFMA's
error bound of each GEMM output, propagated through SwiGLU or its
derivative) plus one grid step of each side; block scales at most one
apart; for the well-conditioned elements (carried error below a quarter
step), every differing code exactly one step apart and a mismatch rate of at
most 1e-3. The rates are printed.
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


def _grid_step(v, scale_code):
    """Spacing of the E4M3 grid (times the block scale) at magnitude |v|."""
    X = orc.e8m0_value(scale_code)
    t = np.abs(v) / X
    _, ex = np.frexp(np.where(t > 0, t, 2.0 ** -10))     # zero lies in the subnormal range
    E = np.maximum(ex.astype(np.int64) - 1, -6)          # binade, subnormals share 2^-6's spacing
    return np.exp2((E - 3).astype(np.float64)) * X


def _compare(tag, q_gpu, s_gpu, q_ref, s_ref, tol):
    """Codes and scales of one layout against the oracle's quantization of its
    own float64 values. tol: per element, a bound on |GPU value - oracle
    value| before quantization (the GEMM error carried through the
    epilogue's arithmetic)."""
    rows, cols = q_ref.shape
    assert q_gpu.shape == q_ref.shape and s_gpu.shape == s_ref.shape, tag
    ds = np.abs(s_gpu.astype(np.int64) - s_ref.astype(np.int64))
    assert ds.max() <= 1, f"{tag}: a block scale differs by {ds.max()}"
    sg = np.repeat(s_gpu, 32, axis=1)
    so = np.repeat(s_ref, 32, axis=1)
    vg = orc.e4m3_value(q_gpu) * orc.e8m0_value(sg)
    vo = orc.e4m3_value(q_ref) * orc.e8m0_value(so)
    # each side rounds its value once to its own block's grid (at most half a
    # step each); the values themselves differ by at most tol
    lim = tol + _grid_step(vg, sg) + _grid_step(vo, so)
    err = np.abs(vg - vo)
    worst = float(np.max(err / np.maximum(lim, 1e-300)))
    assert np.all(err <= lim), f"{tag}: a value differs by {worst:.2f}x its bound"
    mis = q_gpu != q_ref
    same = (ds == 0).repeat(32, axis=1)
    # well-conditioned elements (carried error below a quarter step, same
    # scale): codes equal or one step apart, rarely apart
    wc = same & (tol < 0.25 * _grid_step(vo, so))
    steps = np.abs(_grid_index(q_gpu) - _grid_index(q_ref))
    assert np.all(steps[wc] <= 1), f"{tag}: a well-conditioned code differs by {int(steps[wc].max())} steps"
    rate_wc = float(np.mean(mis[wc])) if wc.any() else 0.0
    print(f"[intermediates] {tag}: code mismatch rate {np.mean(mis):.2e} over {mis.size} codes; well-conditioned "
          f"{np.mean(wc):.3f} of them, mismatch rate {rate_wc:.2e} (all one step); "
          f"{int((ds > 0).sum())} of {ds.size} block scales one apart; worst |diff| / bound {worst:.3f}", flush=True)
    assert rate_wc <= MAX_RATE, f"{tag}: well-conditioned mismatch rate {rate_wc}"
    return rate_wc


def _silu_prime(g):
    s = orc.sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def _silu_second(g):
    s = orc.sigmoid(g)
    return s * (1.0 - s) * (2.0 + g * (1.0 - 2.0 * s))


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
    dyh = orc.dequantize_rowwise(*orc.quantize_rowwise(orc.bf16_bits_to_f64(c["dy"])))
    off = np.concatenate([[0], np.cumsum(split)])
    bound_h1 = np.zeros((R, 2 * F))       # |fp32 GEMM - float64| of H1
    bound_da = np.zeros((R, F))           # same for dA = dY . columnwise(W2)
    for e in range(E):
        if split[e]:
            r = slice(off[e], off[e + 1])
            w1h = orc.dequantize_rowwise(*orc.quantize_rowwise(orc.bf16_bits_to_f64(c["w1"][e])))
            bound_h1[r] = mfma_gemm_bound(xh[r], w1h)
            q2, s2 = orc.quantize_colwise(orc.bf16_bits_to_f64(c["w2"][e]))       # [F, H]
            bound_da[r] = mfma_gemm_bound(dyh[r], orc.dequantize_rowwise(q2, s2))
    dh = np.abs(h1_gpu - fwd["h1_bf16"])
    lim_h1 = bound_h1 + 2.0 ** -8 * (np.abs(fwd["h1"]) + np.abs(h1_gpu))
    assert np.all(dh <= lim_h1), f"H1 off by {float(np.max(dh / np.maximum(lim_h1, 1e-300))):.2f}x the bound"
    print(f"[intermediates] {name}: H1 bf16 differs at a rate of {np.mean(dh > 0):.2e}", flush=True)

    w = c["probs"].astype(np.float64)[:, None]
    g, u = fwd["h1"][:, :F], fwd["h1"][:, F:]
    # A = w silu(g) u from fp32 accumulators: carried error of the GEMM
    tol_a = 2.0 * w * (np.abs(_silu_prime(g) * u) * bound_h1[:, :F] + np.abs(orc.silu(g)) * bound_h1[:, F:])
    # dH1 from dA (GEMM error) and the bf16 H1 (the two sides' bf16 H1 differ
    # by at most lim_h1)
    gb, ub, da = fwd["h1_bf16"][:, :F], fwd["h1_bf16"][:, F:], bwd["da"]
    dg_, du_ = lim_h1[:, :F], lim_h1[:, F:]
    tol_dg = 2.0 * w * (np.abs(ub * _silu_prime(gb)) * bound_da + np.abs(da * _silu_prime(gb)) * du_
                        + np.abs(da * ub * _silu_second(gb)) * dg_)
    tol_du = 2.0 * w * (np.abs(orc.silu(gb)) * bound_da + np.abs(da * _silu_prime(gb)) * dg_)
    tol_dh = np.concatenate([tol_dg, tol_du], axis=1)

    def colwise_tol(t):
        """The [rows, cols] tolerance in the grouped columnwise layout [cols, sumP]."""
        out = np.zeros((t.shape[1], P))
        p0 = 0
        for e in range(E):
            out[:, p0:p0 + split[e]] = t[off[e]:off[e + 1]].T
            p0 += (split[e] + 31) // 32 * 32
        return out

    # A: rowwise [R, F] and grouped columnwise [F, sumP]
    a_q = _bytes(runner.fwd_ws, o["a_row_codes"], R * F).reshape(R, F)
    a_s = _untile_rowwise(_bytes(runner.fwd_ws, o["a_row_scales"], R32 * F // 32), R, F)
    rq, rs = orc.quantize_rowwise(fwd["a"])
    _compare(f"{name} A rowwise", a_q, a_s, rq, rs, tol_a)
    ac_q = _bytes(runner.saved, o["a_col_codes"], F * P).reshape(F, P)
    ac_s = _untile_colwise(_bytes(runner.saved, o["a_col_scales"], F // 32 * nq * 128), F, split, nq)
    cq, cs = orc.quantize_colwise(fwd["a"], split)
    _compare(f"{name} A columnwise", ac_q, ac_s, cq, cs, colwise_tol(tol_a))

    # dH1: rowwise [R, 2F] and grouped columnwise [2F, sumP]
    d_q = _bytes(runner.bwd_ws, o["dh1_row_codes"], R * 2 * F).reshape(R, 2 * F)
    d_s = _untile_rowwise(_bytes(runner.bwd_ws, o["dh1_row_scales"], R32 * 2 * F // 32), R, 2 * F)
    rq, rs = orc.quantize_rowwise(bwd["dh1"])
    _compare(f"{name} dH1 rowwise", d_q, d_s, rq, rs, tol_dh)
    dc_q = _bytes(runner.bwd_ws, o["dh1_col_codes"], 2 * F * P).reshape(2 * F, P)
    dc_s = _untile_colwise(_bytes(runner.bwd_ws, o["dh1_col_scales"], 2 * F // 32 * nq * 128), 2 * F, split, nq)
    cq, cs = orc.quantize_colwise(bwd["dh1"], split)
    _compare(f"{name} dH1 columnwise", dc_q, dc_s, cq, cs, colwise_tol(tol_dh))

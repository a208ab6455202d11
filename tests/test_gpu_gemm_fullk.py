"""Each of the six GEMMs of the fused MLP at its full contraction length, on
the Mixtral-8x7B-shaped forward+backward workload's own operands (4096
tokens, top-2 of 8, H=4096, F=14336), quantized by the oracle on the CPU and
multiplied by mx_grouped_gemm with fp32 output against the oracle's float64
product of the same codes (GroupedLinear over split_sizes and the fused MLP's
GEMMs: "Efficient MoE training for biological foundation models", Key
technical approaches items 1 and 3).

The operands are those of the largest expert: 128 of its rows as the A side
of the group-M GEMMs (K = 4096, 14336, 4096, 28672) and 256 rows (of W1, W2
or their columnwise copies) as the B side; for the group-K wgrads, 256 and
128 columns of its columnwise copies over all its rows (K = its padded row
count). Intermediates (A, dA, dH1) are the oracle's float64 values from the
same inputs.

Assertion: every element within the MFMA's own error bound
(tests.gpu_util.mfma_gemm_bound). The normwise relative error of each GEMM is
printed; NORMWISE_BAR asserts 1e-5 for the GEMMs whose measured error meets
it (None: printed only)."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_u8, mfma_gemm_bound, rel_norm

pytestmark = pytest.mark.gpu
ROWS_A, ROWS_B = 128, 256
# normwise bar per GEMM: 1e-5 where the measured error meets it; where the
# MFMA's alignment loss (about 2^-13 of each 16-product group's largest term)
# sets a higher floor, None, and only the elementwise bound is asserted
NORMWISE_BAR = {"gemm1": None, "gemm2": None, "dgrad2": None, "dgrad1": None, "wgrad2": None, "wgrad1": None}


def _operands():
    w = wl.WORKLOADS["mixtral_moe_fwd_bwd"]
    print("[fullk] generating the workload's inputs", flush=True)
    c = wl.make_mlp_inputs(w, with_dy=True)
    split = c["split_sizes"].astype(np.int64)
    e = int(np.argmax(split))
    off = np.concatenate([[0], np.cumsum(split)])
    r0, r1 = int(off[e]), int(off[e + 1])
    m = r1 - r0
    F, H = w.ffn, w.hidden
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(np.arange(r0, r1), ROWS_A, replace=False))
    x_all = orc.bf16_bits_to_f64(c["x"][r0:r1])
    dy_all = orc.bf16_bits_to_f64(c["dy"][r0:r1])
    w1 = orc.bf16_bits_to_f64(c["w1"][e])            # [2F, H]
    w2 = orc.bf16_bits_to_f64(c["w2"][e])            # [H, F]
    p = c["probs"][r0:r1].astype(np.float64)
    sel = rows - r0
    f_sel = np.sort(rng.choice(F, ROWS_B // 2, replace=False))
    n_sel = np.concatenate([f_sel, F + f_sel])       # gate and up rows of the same ffn columns
    h_sel = np.sort(rng.choice(H, ROWS_B, replace=False))
    ops = {}

    print("[fullk] oracle: quantize W1 rowwise, W2 columnwise", flush=True)
    w1_q, w1_s = orc.quantize_rowwise(w1)
    w1h = orc.dequantize_rowwise(w1_q, w1_s)
    w2c_q, w2c_s = orc.quantize_colwise(w2)          # [F, H]
    w2c = orc.dequantize_rowwise(w2c_q, w2c_s)       # columnwise W2 as [F, H]
    xq, xs = orc.quantize_rowwise(x_all[sel])
    ops["gemm1"] = (xq, xs, w1_q[n_sel], w1_s[n_sel], None)

    # forward intermediates of the sampled rows: H1 -> A (float64, R8)
    h1 = orc.dequantize_rowwise(xq, xs) @ w1h.T      # [128, 2F]
    a = p[sel, None] * orc.silu(h1[:, :F]) * h1[:, F:]
    aq, as_ = orc.quantize_rowwise(a)
    ops["gemm2"] = (aq, as_) + orc.quantize_rowwise(w2[h_sel]) + (None,)

    # dgrad2: rowwise dY x columnwise W2 (rows f of the [F, H] copy)
    dyq, dys = orc.quantize_rowwise(dy_all[sel])
    f_b = np.sort(rng.choice(F, ROWS_B, replace=False))
    ops["dgrad2"] = (dyq, dys, w2c_q[f_b], w2c_s[f_b], None)

    # dgrad1: rowwise dH1 (from dA and the bf16 H1) x columnwise W1 (rows h of the [H, 2F] copy)
    da = orc.dequantize_rowwise(dyq, dys) @ w2c.T    # [128, F]
    hb = orc.round_to_bf16(h1)
    s = orc.sigmoid(hb[:, :F])
    dg = da * p[sel, None] * hb[:, F:] * s * (1 + hb[:, :F] * (1 - s))
    du = da * p[sel, None] * hb[:, :F] * s
    dhq, dhs = orc.quantize_rowwise(np.concatenate([dg, du], axis=1))
    w1c_q, w1c_s = orc.quantize_colwise(w1[:, h_sel])   # [256, 2F]
    ops["dgrad1"] = (dhq, dhs, w1c_q, w1c_s, None)

    # wgrad2: columnwise dY (h columns) x columnwise A (f columns) over all m rows of the expert
    print("[fullk] oracle: expert-wide columns for the weight gradients", flush=True)
    xq_all = orc.dequantize_rowwise(*orc.quantize_rowwise(x_all))
    g_c, u_c = xq_all @ w1h[f_sel].T, xq_all @ w1h[F + f_sel].T
    a_c = p[:, None] * orc.silu(g_c) * u_c
    ops["wgrad2"] = orc.quantize_colwise(dy_all[:, h_sel[:ROWS_A]]) + orc.quantize_colwise(a_c) + (m,)

    # wgrad1: columnwise dH1 (n columns: the gate and up of f_sel) x columnwise X (h columns)
    dyq_all = orc.dequantize_rowwise(*orc.quantize_rowwise(dy_all))
    da_c = dyq_all @ w2c[f_sel].T
    gb, ub = orc.round_to_bf16(g_c), orc.round_to_bf16(u_c)
    s_c = orc.sigmoid(gb)
    dg_c = da_c * p[:, None] * ub * s_c * (1 + gb * (1 - s_c))
    du_c = da_c * p[:, None] * gb * s_c
    dh_c = np.concatenate([dg_c[:, :ROWS_A // 2], du_c[:, :ROWS_A // 2]], axis=1)
    ops["wgrad1"] = orc.quantize_colwise(dh_c) + orc.quantize_colwise(x_all[:, h_sel]) + (m,)
    return ops


@pytest.fixture(scope="module")
def fullk_ops():
    return _operands()


@pytest.mark.parametrize("gemm", ["gemm1", "gemm2", "dgrad2", "dgrad1", "wgrad2", "wgrad1"])
def test_gemm_full_contraction_on_workload_operands(gpu_lib, fullk_ops, gemm):
    aq, as_, bq, bs, m = fullk_ops[gemm]
    M, K = aq.shape
    N = bq.shape[0]
    assert bq.shape[1] == K
    if m is None:
        c = gpu_lib.grouped_gemm(gpu_lib.MX_GROUP_M, [M], dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs),
                                 N=N, K=K)
    else:        # group-K: one group of m rows, padded to K
        c = gpu_lib.grouped_gemm(gpu_lib.MX_GROUP_K, [m], dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs),
                                 N=N, K=K)[0]
    torch.cuda.synchronize()
    got = c.cpu().numpy().astype(np.float64)
    A = orc.dequantize_rowwise(aq, as_)
    B = orc.dequantize_rowwise(bq, bs)
    want = A @ B.T
    bound = mfma_gemm_bound(A, B)
    err = np.abs(got - want)
    rn = rel_norm(got, want)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    print(f"[fullk] {gemm}: M={M} N={N} K={K} normwise {rn:.3e}, worst error / MFMA bound {worst:.3f}", flush=True)
    assert np.all(err <= bound), f"{gemm}: error exceeds the MFMA bound ({worst:.2f}x)"
    if NORMWISE_BAR[gemm] is not None:
        assert rn <= NORMWISE_BAR[gemm], f"{gemm}: normwise {rn:.3e} above {NORMWISE_BAR[gemm]:.0e}"

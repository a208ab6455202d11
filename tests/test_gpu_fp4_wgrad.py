"""GPU parity of the grouped columnwise MXFP4 cast and the MXFP4 weight-
gradient GEMM (reading R16) against the oracle.

Cast: codes and scales bit-exact, over groups that are empty, one row, just
under and over 32 and 128 rows. GEMM: with scale codes 126..128 and at most
256 values per group every partial sum is a multiple of 2^-4 below 2^16, so
the fp32 result must equal the oracle exactly whatever the summation order
(groups whose padded range ends half-way into a 64-value MFMA step, whose
other half holds the next group's codes, are included: their scales are
zeroed on both operands); accumulation adds into starting values that are
multiples of 2^-4, again exactly; wide scales are checked against the MFMA
error bound. Canary bytes around C catch stores outside it."""
import numpy as np
import pytest
import torch

import oracle as orc
from tests.gpu_util import canaries_intact, dev_bf16, dev_u8, guarded, mfma_gemm_bound, to_np
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sizes,cols", [((0, 1, 31, 33, 128, 129, 300, 0), 96), ((64,), 32), ((5, 250), 4096)])
def test_grouped_colwise_cast_bit_exact(gpu_lib, sizes, cols):
    rng = np.random.default_rng(400 + sum(sizes))
    R = sum(sizes)
    x = rng.standard_t(3, size=(R, cols)) * np.exp2(rng.integers(-12, 12, size=(1, cols)))
    if R:
        x[rng.random(R) < 0.1] = 0.0
    xb = wl.bf16_bits_from_f32(x.astype(np.float32))
    qc, sc = gpu_lib.mx_quantize_fp4_colwise_grouped(dev_bf16(xb), sizes)
    torch.cuda.synchronize()
    wq, ws = orc.quantize_colwise_fp4(orc.bf16_bits_to_f64(xb), sizes)
    assert np.array_equal(sc.cpu().numpy(), ws)
    assert np.array_equal(qc.cpu().numpy(), wq)


def _operand(rng, rows, K, lo, hi):
    return (rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8),
            rng.integers(lo, hi + 1, size=(rows, K // 32), dtype=np.uint8))


def _wgrad(mx, aq, as_, bq, bs, sizes, init=None):
    G, m, n = len(sizes), aq.shape[0], bq.shape[0]
    buf, c = guarded((G, m, n), torch.float32)
    if init is not None:
        c.copy_(torch.from_numpy(init.astype(np.float32)).cuda())
    mx.mx_grouped_gemm_fp4_wgrad(dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs), sizes, out=c,
                                 accumulate=init is not None)
    torch.cuda.synchronize()
    assert canaries_intact(buf), "the wgrad GEMM wrote outside C"
    return to_np(c)


@pytest.mark.parametrize("sizes,m,n", [((20, 0, 64, 33, 96, 250), 300, 130), ((1,), 1, 1), ((256, 200), 256, 256)])
def test_wgrad_exact(gpu_lib, sizes, m, n):
    rng = np.random.default_rng(500 + m)
    K = int(orc.padded_sizes(sizes).sum())
    aq, as_ = _operand(rng, m, K, 126, 128)
    bq, bs = _operand(rng, n, K, 126, 128)
    want = orc.gemm_fp4_group_k(aq, as_, bq, bs, sizes)
    got = _wgrad(gpu_lib, aq, as_, bq, bs, sizes)
    assert np.array_equal(got, want), f"max |diff| {np.max(np.abs(got - want))}"
    init = rng.integers(-2 ** 14, 2 ** 14, size=want.shape) / 16.0
    got = _wgrad(gpu_lib, aq, as_, bq, bs, sizes, init=init)
    assert np.array_equal(got, init + want), "accumulate"


def test_wgrad_wide_scales_within_bound(gpu_lib):
    rng = np.random.default_rng(600)
    sizes = [700, 0, 1100, 33, 248]
    m, n = 384, 320
    K = int(orc.padded_sizes(sizes).sum())
    aq, as_ = _operand(rng, m, K, 120, 134)
    bq, bs = _operand(rng, n, K, 120, 134)
    want = orc.gemm_fp4_group_k(aq, as_, bq, bs, sizes)
    got = _wgrad(gpu_lib, aq, as_, bq, bs, sizes)
    A = orc.dequantize_rowwise_fp4(aq, as_)
    B = orc.dequantize_rowwise_fp4(bq, bs)
    k0 = 0
    for g, p in enumerate(orc.padded_sizes(sizes).tolist()):
        if p:
            bound = mfma_gemm_bound(A[:, k0:k0 + p], B[:, k0:k0 + p])
            assert np.all(np.abs(got[g] - want[g]) <= bound), f"group {g}"
        else:
            assert np.all(got[g] == 0)
        k0 += p


def test_wgrad_of_gpu_cast_activations(gpu_lib):
    """End to end on the device: both routed activations cast by the grouped
    columnwise MXFP4 cast, then the wgrad GEMM; against the oracle's product
    of the oracle's own casts (bit-identical by the cast test above)."""
    rng = np.random.default_rng(700)
    sizes = [300, 0, 129, 64]
    R, m, n = sum(sizes), 256, 192
    xa = wl.bf16_bits_from_f32((rng.standard_normal((R, m)) * 1e-2).astype(np.float32))
    xb = wl.bf16_bits_from_f32(rng.standard_normal((R, n)).astype(np.float32))
    aq, as_ = gpu_lib.mx_quantize_fp4_colwise_grouped(dev_bf16(xa), sizes)
    bq, bs = gpu_lib.mx_quantize_fp4_colwise_grouped(dev_bf16(xb), sizes)
    got = to_np(gpu_lib.mx_grouped_gemm_fp4_wgrad(aq, as_, bq, bs, sizes))
    oaq, oas = orc.quantize_colwise_fp4(orc.bf16_bits_to_f64(xa), sizes)
    obq, obs = orc.quantize_colwise_fp4(orc.bf16_bits_to_f64(xb), sizes)
    want = orc.gemm_fp4_group_k(oaq, oas, obq, obs, sizes)
    A, B = orc.dequantize_rowwise_fp4(oaq, oas), orc.dequantize_rowwise_fp4(obq, obs)
    k0 = 0
    for g, p in enumerate(orc.padded_sizes(sizes).tolist()):
        if p:
            assert np.all(np.abs(got[g] - want[g]) <= mfma_gemm_bound(A[:, k0:k0 + p], B[:, k0:k0 + p]))
        k0 += p


def test_wgrad_mixtral_sampled(gpu_lib):
    """The Mixtral MLP's first weight gradient at MXFP4: dW1[e] = dH[e]^T X[e]
    over 8192 routed rows of 8 experts (ragged, one empty), m = 2 x 14336,
    n = 4096; sampled rows and columns of every expert's block, each against
    the oracle's dot product of that expert's padded k range."""
    rng = np.random.default_rng(800)
    sizes = [157, 574, 1914, 3333, 0, 1562, 71, 581]
    m, n, G = 28672, 4096, len(sizes)
    pad = orc.padded_sizes(sizes)
    K = int(pad.sum())
    aq, as_ = _operand(rng, m, K, 122, 132)
    bq, bs = _operand(rng, n, K, 122, 132)
    c = gpu_lib.mx_grouped_gemm_fp4_wgrad(dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs), sizes)
    torch.cuda.synchronize()
    k0 = np.concatenate([[0], np.cumsum(pad)])
    for g in range(G):
        rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 6)]))
        cols = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 60)]))
        got = to_np(c[g][torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
        if pad[g] == 0:
            assert np.all(got == 0), f"expert {g} (empty)"
            continue
        ks = slice(int(k0[g]) // 2, int(k0[g + 1]) // 2)
        ss = slice(int(k0[g]) // 32, int(k0[g + 1]) // 32)
        A = orc.dequantize_rowwise_fp4(aq[rows][:, ks], as_[rows][:, ss])
        B = orc.dequantize_rowwise_fp4(bq[cols][:, ks], bs[cols][:, ss])
        assert np.all(np.abs(got - A @ B.T) <= mfma_gemm_bound(A, B)), f"expert {g}"

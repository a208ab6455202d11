"""GPU parity of the NVFP4 cast and GEMMs against the oracle (reading R18: E2M1
elements, one E4M3 scale per 16 values, one fp32 scale per tensor; the NVFP4
recipe of "TransformerEngine-accelerated Llama 3 training with native PyTorch
training loop", Quantized Training).

Cast: codes, block scales and amax bit-exact (both sides take every decision
in fp32 with the same steps), on ragged shapes, zero blocks, blocks that
flush to zero, the hand-worked tie block of the oracle pins, and sampled rows
of the Mixtral-sized activation.

GEMM: with block scales 1 .. 1.875 (E4M3 codes 0x38 .. 0x3F), tensor scale 1
(amax 2688) and k <= 384 every element is a multiple of 1/16 below 12, every
product a multiple of 1/256 and every partial sum below 2^24 / 256, so the
fp32 result must equal the oracle exactly, whatever the summation order; a
bf16 result is its nearest-even rounding. Elsewhere the bar is the fp32
summation bound k * 2^-23 * sum |a b| plus one rounding of the tensor-scale
factor and, for bf16 output, half a bf16 step."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import dev_bf16, dev_u8, to_np

pytestmark = pytest.mark.gpu


def _cast_input(rng, rows, cols, spread=8, zero_frac=0.1):
    x = rng.standard_t(3, size=(rows, cols)) * np.exp2(rng.integers(-spread, spread, size=(rows, cols // 16))).repeat(16, axis=1)
    if rows and zero_frac:
        z = rng.random((rows, cols // 16)) < zero_frac
        x[z.repeat(16, axis=1)] = 0.0
    return wl.bf16_bits_from_f32(x.astype(np.float32))


def _check_cast(gpu_lib, xb, colwise):
    x = orc.bf16_bits_to_f64(xb)
    out = gpu_lib.mx_quantize_nvfp4(dev_bf16(xb), colwise=colwise)
    torch.cuda.synchronize()
    q, s, amax = orc.quantize_rowwise_nvfp4(x)
    assert np.float32(out[2].item()) == amax
    assert np.array_equal(out[1].cpu().numpy(), s), "block scales"
    assert np.array_equal(out[0].cpu().numpy(), q), "codes"
    if colwise:
        qc, sc, _ = orc.quantize_colwise_nvfp4(x)
        assert np.array_equal(out[4].cpu().numpy(), sc), "columnwise block scales"
        assert np.array_equal(out[3].cpu().numpy(), qc), "columnwise codes"


@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 80), (144, 208), (304, 4096)])
def test_nvfp4_cast_bit_exact(gpu_lib, rows, cols):
    rng = np.random.default_rng(900 + rows + cols)
    _check_cast(gpu_lib, _cast_input(rng, rows, cols), colwise=True)


def test_nvfp4_cast_wide_spread_flushes_and_ties(gpu_lib):
    """Block maxima over 40 binades (E4M3 scales flush the small blocks) and
    row 0 = the oracle pins' hand-worked blocks (S = 1, float32 ties)."""
    rng = np.random.default_rng(950)
    xb = _cast_input(rng, 64, 256, spread=20, zero_frac=0.0)
    row = np.zeros(256)
    row[0] = 2688.0
    row[16:24] = [9, 4.5, 2.25, 1.0, 0.375, 0.75, 3.75, -9]
    row[32:35] = [6, -3, 1.25]
    xb[0] = wl.bf16_bits_from_f32(row.astype(np.float32))
    xb[1:] = wl.bf16_bits_from_f32((orc.bf16_bits_to_f64(xb[1:]) * 1e-3).astype(np.float32))   # row 0 holds amax
    _check_cast(gpu_lib, xb, colwise=True)


def test_nvfp4_cast_zero_tensor(gpu_lib):
    xb = np.zeros((32, 64), dtype=np.uint16)
    xb[5, 7] = 0x8000                                                  # -0
    _check_cast(gpu_lib, xb, colwise=True)


def test_nvfp4_cast_full_size_sampled(gpu_lib):
    """The Mixtral-sized activation (8192 x 4096): amax over the whole tensor,
    sampled rows and columns bit-exact."""
    rng = np.random.default_rng(960)
    xb = _cast_input(rng, 8192, 4096, spread=6)
    q, s, amax, qc, sc = gpu_lib.mx_quantize_nvfp4(dev_bf16(xb), colwise=True)
    torch.cuda.synchronize()
    x = orc.bf16_bits_to_f64(xb)
    want_amax = np.float32(np.max(np.abs(x)))
    assert np.float32(amax.item()) == want_amax
    rows = np.unique(np.concatenate([[0, 8191], rng.integers(0, 8192, 14)]))
    wq, ws, _ = orc.quantize_rowwise_nvfp4(x[rows], amax=want_amax)
    assert np.array_equal(q.cpu().numpy()[rows], wq) and np.array_equal(s.cpu().numpy()[rows], ws)
    cols = np.unique(np.concatenate([[0, 4095], rng.integers(0, 4096, 14)]))
    wqc, wsc, _ = orc.quantize_rowwise_nvfp4(x[:, cols].T, amax=want_amax)
    assert np.array_equal(qc.cpu().numpy()[cols], wqc) and np.array_equal(sc.cpu().numpy()[cols], wsc)


def _operand(rng, rows, k, lo=0x38, hi=0x3F):
    return (rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8),
            rng.integers(lo, hi + 1, size=(rows, k // 16), dtype=np.uint8))


def _f32(v):
    return torch.tensor(np.asarray(v, dtype=np.float32).reshape(-1), device="cuda")


@pytest.mark.parametrize("sizes,n,k", [((300,), 130, 256), ((100, 0, 200), 256, 384), ((1,), 1, 128),
                                       ((257, 33, 0, 190), 300, 256)])
def test_nvfp4_gemm_exact(gpu_lib, sizes, n, k):
    rng = np.random.default_rng(970 + n + k)
    m, G = sum(sizes), len(sizes)
    aq, as_ = _operand(rng, m, k)
    bq = rng.integers(0, 256, size=(G, n, k // 2), dtype=np.uint8)
    bs = rng.integers(0x38, 0x40, size=(G, n, k // 16), dtype=np.uint8)
    amax = np.float32(2688.0)
    want = orc.gemm_nvfp4_grouped(aq, as_, amax, bq, bs, np.full(G, amax, np.float32), sizes)
    for dt in (torch.float32, torch.bfloat16):
        got = gpu_lib.mx_grouped_gemm_nvfp4(dev_u8(aq), dev_u8(as_), _f32(amax), dev_u8(bq), dev_u8(bs),
                                            _f32(np.full(G, amax)), sizes, out_dtype=dt)
        torch.cuda.synchronize()
        exp = want if dt == torch.float32 else orc.round_to_bf16(want)
        assert np.array_equal(to_np(got), exp), f"{dt}: max |diff| {np.max(np.abs(to_np(got) - exp))}"


def _bound(A, B, want, bf16):
    k = A.shape[1]
    b = k * 2.0 ** -23 * (np.abs(A) @ np.abs(B).T) + 2.0 ** -22 * np.abs(want)
    return b + (2.0 ** -8 * np.abs(want) if bf16 else 0)


def test_nvfp4_gemm_of_gpu_casts_with_per_group_scales(gpu_lib):
    """GPU casts of an activation and of three expert weights (each its own
    tensor scale), then the grouped GEMM; the casts are bit-exact against the
    oracle's (tests above), so the GEMM is compared with the oracle's product
    of the oracle's casts."""
    rng = np.random.default_rng(980)
    sizes = [150, 0, 300]
    m, k, n = sum(sizes), 512, 192
    xb = _cast_input(rng, m, k, spread=3)
    ws = [_cast_input(rng, n, k, spread=2) for _ in sizes]
    ws[2] = wl.bf16_bits_from_f32((orc.bf16_bits_to_f64(ws[2]) * 300.0).astype(np.float32))
    aq, as_, aa = gpu_lib.mx_quantize_nvfp4(dev_bf16(xb))
    casts = [gpu_lib.mx_quantize_nvfp4(dev_bf16(w)) for w in ws]
    bq = torch.stack([c[0] for c in casts])
    bs = torch.stack([c[1] for c in casts])
    ba = torch.cat([c[2] for c in casts])
    got = to_np(gpu_lib.mx_grouped_gemm_nvfp4(aq, as_, aa, bq, bs, ba, sizes, out_dtype=torch.float32))
    oa = orc.quantize_rowwise_nvfp4(orc.bf16_bits_to_f64(xb))
    ob = [orc.quantize_rowwise_nvfp4(orc.bf16_bits_to_f64(w)) for w in ws]
    assert ob[0][2] != ob[2][2]
    want = orc.gemm_nvfp4_grouped(oa[0], oa[1], oa[2], np.stack([o[0] for o in ob]), np.stack([o[1] for o in ob]),
                                  np.array([o[2] for o in ob], np.float32), sizes)
    A = orc.dequantize_rowwise_nvfp4(*oa)
    r0 = 0
    for g, msz in enumerate(sizes):
        if msz:
            B = orc.dequantize_rowwise_nvfp4(*ob[g])
            sl = slice(r0, r0 + msz)
            assert np.all(np.abs(got[sl] - want[sl]) <= _bound(A[sl], B, want[sl], False)), f"group {g}"
        r0 += msz


def test_nvfp4_gemm_mixtral_sampled(gpu_lib):
    """The Mixtral MLP's first GEMM at NVFP4: 8192 routed rows over 8 experts
    (ragged), n = 28672, k = 4096, bf16 out, random codes and E4M3 scales
    (0x20 .. 0x50) with per-expert tensor scales; sampled rows of every expert
    against the oracle's dot products."""
    rng = np.random.default_rng(990)
    sizes = [157, 574, 1914, 3333, 1056, 506, 71, 581]
    m, n, k, G = sum(sizes), 28672, 4096, len(sizes)
    aq, as_ = _operand(rng, m, k, 0x20, 0x50)
    bq = rng.integers(0, 256, size=(G, n, k // 2), dtype=np.uint8)
    bs = rng.integers(0x20, 0x51, size=(G, n, k // 16), dtype=np.uint8)
    a_amax = np.float32(3.25)
    b_amax = (rng.uniform(0.01, 2.0, size=G)).astype(np.float32)
    c = gpu_lib.mx_grouped_gemm_nvfp4(dev_u8(aq), dev_u8(as_), _f32(a_amax), dev_u8(bq), dev_u8(bs), _f32(b_amax),
                                      sizes)
    torch.cuda.synchronize()
    row0 = np.concatenate([[0], np.cumsum(sizes)])
    cols = np.sort(rng.choice(n, 128, replace=False))
    for g in range(G):
        rows = np.unique(np.concatenate([[row0[g], row0[g + 1] - 1], rng.integers(row0[g], row0[g + 1], 4)]))
        got = to_np(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
        A = orc.dequantize_rowwise_nvfp4(aq[rows], as_[rows], a_amax)
        B = orc.dequantize_rowwise_nvfp4(bq[g][cols], bs[g][cols], b_amax[g])
        want = A @ B.T
        assert np.all(np.abs(got - want) <= _bound(A, B, want, True)), f"expert {g}"

"""GPU parity of the rowwise MXFP4 cast (mx_quantize_fp4) against the oracle
(reading R14): codes and scales bit-exact, on every finite bf16 value in
blocks whose amax is 2^(k+d) for d = 0..6 (every element/scale ratio the
E2M1 grid distinguishes, including all ties), on ragged random tensors with
zero blocks, and on the 16384 x 4096 Student-t tensor (sampled rows)."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import canaries_intact, dev_bf16, dev_u8, guarded, mfma_gemm_bound, rel_norm, to_np

pytestmark = pytest.mark.gpu


def _cast(mx, bits):
    q, s = mx.mx_quantize_fp4(dev_bf16(bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def test_fp4_exhaustive_bf16_times_scales(gpu_lib):
    bits = np.arange(65536, dtype=np.uint32)
    ef = (bits >> 7) & 0xFF
    bits = bits[(ef != 0xFF) & ((bits & 0x7FFF) != 0)].astype(np.uint16)
    v = orc.bf16_bits_to_f64(bits)
    _, ex = np.frexp(np.abs(v))
    k = ex.astype(np.int64) - 1
    blocks = []
    for d in range(0, 7):
        keep = k + d <= 127
        b = np.zeros((int(keep.sum()), 32))
        b[:, 0] = v[keep]
        b[:, 7] = np.ldexp(1.0, k[keep] + d)
        blocks.append(b)
    x = np.concatenate(blocks)
    xb = wl.bf16_bits_from_f32(x.astype(np.float32))
    assert np.array_equal(orc.bf16_bits_to_f64(xb), x)
    q, s = _cast(gpu_lib, xb)
    wq, ws = orc.quantize_rowwise_fp4(x)
    assert np.array_equal(s, ws)
    assert np.array_equal(q, wq)


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (300, 4096)])
def test_fp4_random_with_zero_blocks(gpu_lib, rows, cols):
    rng = np.random.default_rng(90 + rows)
    x = rng.standard_t(3, size=(rows, cols)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))
    x[:, :32][rng.random(rows) < 0.2] = 0.0
    xb = wl.bf16_bits_from_f32(x.astype(np.float32))
    q, s = _cast(gpu_lib, xb)
    wq, ws = orc.quantize_rowwise_fp4(orc.bf16_bits_to_f64(xb))
    assert np.array_equal(s, ws) and np.array_equal(q, wq)


def test_fp4_full_size_sampled(gpu_lib):
    bits = wl.quantize_tensor_c2()
    q, s = _cast(gpu_lib, bits)
    rows = np.random.default_rng(1).choice(bits.shape[0], size=256, replace=False)
    wq, ws = orc.quantize_rowwise_fp4(orc.bf16_bits_to_f64(bits[rows]))
    assert np.array_equal(s[rows], ws) and np.array_equal(q[rows], wq)


@pytest.mark.parametrize("rows,cols", [(32, 32), (96, 160), (384, 4096)])
def test_fp4_colwise_is_rowwise_of_transpose(gpu_lib, rows, cols):
    """The columnwise copy equals the oracle's rowwise MXFP4 of x transposed,
    with ragged column tiles and zero blocks; the rowwise pair of the same
    call is unchanged."""
    rng = np.random.default_rng(95 + rows)
    x = rng.standard_t(3, size=(rows, cols)) * np.exp2(rng.integers(-10, 10, size=(1, cols)))
    x[:32, rng.random(cols) < 0.2] = 0.0
    xb = wl.bf16_bits_from_f32(x.astype(np.float32))
    q, s, qc, sc = gpu_lib.mx_quantize_fp4(dev_bf16(xb), colwise=True)
    torch.cuda.synchronize()
    xf = orc.bf16_bits_to_f64(xb)
    wq, ws = orc.quantize_rowwise_fp4(xf)
    wqc, wsc = orc.quantize_rowwise_fp4(xf.T)
    assert np.array_equal(q.cpu().numpy(), wq) and np.array_equal(s.cpu().numpy(), ws)
    assert np.array_equal(sc.cpu().numpy(), wsc)
    assert np.array_equal(qc.cpu().numpy(), wqc)


def test_fp4_colwise_full_size_sampled(gpu_lib):
    # both layouts in one call (one pass over x): sampled columns of the
    # columnwise copy and sampled rows of the rowwise copy
    bits = wl.quantize_tensor_c2()
    q, s, qc, sc = gpu_lib.mx_quantize_fp4(dev_bf16(bits), colwise=True)
    torch.cuda.synchronize()
    cols = np.random.default_rng(2).choice(bits.shape[1], size=128, replace=False)
    wqc, wsc = orc.quantize_rowwise_fp4(orc.bf16_bits_to_f64(bits[:, cols]).T)
    assert np.array_equal(sc.cpu().numpy()[cols], wsc)
    assert np.array_equal(qc.cpu().numpy()[cols], wqc)
    rows = np.random.default_rng(3).choice(bits.shape[0], size=256, replace=False)
    wq, ws = orc.quantize_rowwise_fp4(orc.bf16_bits_to_f64(bits[rows]))
    assert np.array_equal(s.cpu().numpy()[rows], ws) and np.array_equal(q.cpu().numpy()[rows], wq)


# ---- MXFP4 GEMM (mx_gemm_fp4) against the oracle's gemm_fp4 on the same codes

def _fp4_operand(rng, rows, k, lo, hi):
    """Random MXFP4 operand: every byte value (all 16 codes per nibble, -0
    included) and block scale codes in [lo, hi]."""
    q = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    s = rng.integers(lo, hi + 1, size=(rows, k // 32), dtype=np.uint8)
    return q, s


def _gemm_fp4(mx, aq, as_, bq, bs, dtype):
    m, n = aq.shape[0], bq.shape[0]
    buf, c = guarded((m, n), dtype)
    mx.mx_gemm_fp4(dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs), out=c)
    torch.cuda.synchronize()
    assert canaries_intact(buf), "mx_gemm_fp4 wrote outside C"
    return to_np(c)


@pytest.mark.parametrize("m,n", [(300, 200), (257, 130), (1, 1), (128, 128)])
def test_gemm_fp4_exact(gpu_lib, m, n):
    # scale codes 126..128 and k = 256 keep every partial sum a multiple of
    # 2^-4 below 2^16: the fp32 result is exact whatever the summation order,
    # so any mispaired element, nibble or scale shows as a mismatch
    rng = np.random.default_rng(1000 + m)
    k = 256
    aq, as_ = _fp4_operand(rng, m, k, 126, 128)
    bq, bs = _fp4_operand(rng, n, k, 126, 128)
    got = _gemm_fp4(gpu_lib, aq, as_, bq, bs, torch.float32)
    want = orc.gemm_fp4(aq, as_, bq, bs)
    assert np.array_equal(got, want), f"max |diff| {np.max(np.abs(got - want))}"


@pytest.mark.parametrize("m,n,k", [(257, 130, 512), (96, 300, 64), (512, 256, 1024)])
def test_gemm_fp4_wide_scales_within_bound(gpu_lib, m, n, k):
    # scale codes over 2^-7 .. 2^7: inexact sums, checked against the MFMA's
    # error bound (fp32) and bound plus one bf16 rounding (bf16 output)
    rng = np.random.default_rng(2000 + k)
    aq, as_ = _fp4_operand(rng, m, k, 120, 134)
    bq, bs = _fp4_operand(rng, n, k, 120, 134)
    A = orc.dequantize_rowwise_fp4(aq, as_)
    B = orc.dequantize_rowwise_fp4(bq, bs)
    want = orc.gemm_fp4(aq, as_, bq, bs)
    bound = mfma_gemm_bound(A, B)
    got = _gemm_fp4(gpu_lib, aq, as_, bq, bs, torch.float32)
    assert np.all(np.abs(got - want) <= bound)
    got16 = _gemm_fp4(gpu_lib, aq, as_, bq, bs, torch.bfloat16)
    assert np.all(np.abs(got16 - want) <= bound + 2.0 ** -8 * np.abs(want))
    assert rel_norm(got, want) <= 1e-5


def test_gemm_fp4_of_oracle_cast(gpu_lib):
    # operands cast from normal bf16 data by the oracle's MXFP4 quantizer
    rng = np.random.default_rng(31)
    m, n, k = 384, 320, 768
    a = orc.bf16_bits_to_f64(wl.normal_bf16(rng, (m, k)))
    b = orc.bf16_bits_to_f64(wl.normal_bf16(rng, (n, k), std=0.02))
    aq, as_ = orc.quantize_rowwise_fp4(a)
    bq, bs = orc.quantize_rowwise_fp4(b)
    want = orc.gemm_fp4(aq, as_, bq, bs)
    got = _gemm_fp4(gpu_lib, aq, as_, bq, bs, torch.float32)
    bound = mfma_gemm_bound(orc.dequantize_rowwise_fp4(aq, as_), orc.dequantize_rowwise_fp4(bq, bs))
    assert np.all(np.abs(got - want) <= bound)


def test_gemm_fp4_empty_is_noop(gpu_lib):
    z = torch.empty((0, 32), dtype=torch.uint8, device="cuda")
    zs = torch.empty((0, 2), dtype=torch.uint8, device="cuda")
    bq = torch.zeros((4, 32), dtype=torch.uint8, device="cuda")
    bs = torch.full((4, 2), 127, dtype=torch.uint8, device="cuda")
    out = gpu_lib.mx_gemm_fp4(z, zs, bq, bs)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 4)


def test_gemm_fp4_full_size_sampled(gpu_lib):
    # the shape of the Mixtral MLP's first GEMM as one group at MXFP4: 16384
    # routed rows, 28672 gate and up columns, k = 4096, bf16 output; sampled
    # rows and columns recomputed by the oracle
    m, n, k = 16384, 28672, 4096
    rng = np.random.default_rng(77)
    aq, as_ = _fp4_operand(rng, m, k, 122, 132)
    bq, bs = _fp4_operand(rng, n, k, 122, 132)
    c = gpu_lib.mx_gemm_fp4(dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, m - 1], rng.choice(m, 14, replace=False)]))
    cols = np.sort(np.concatenate([[0, n - 1], rng.choice(n, 254, replace=False)]))
    got = to_np(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    A = orc.dequantize_rowwise_fp4(aq[rows], as_[rows])
    B = orc.dequantize_rowwise_fp4(bq[cols], bs[cols])
    want = A @ B.T
    bound = mfma_gemm_bound(A, B) + 2.0 ** -8 * np.abs(want)
    assert np.all(np.abs(got - want) <= bound)


@pytest.mark.parametrize("sizes", [[300, 0, 1, 257, 64], [0, 513], [17]])
def test_grouped_gemm_fp4_exact(gpu_lib, sizes):
    # GroupedLinear at MXFP4: ragged groups (an empty one, a single row, tails
    # inside a 256-row tile), per-group weights; exact regime as above, fp32
    # out, canaries around C
    rng = np.random.default_rng(3000 + len(sizes))
    m, n, k, G = sum(sizes), 200, 256, len(sizes)
    aq, as_ = _fp4_operand(rng, m, k, 126, 128)
    bq = rng.integers(0, 256, size=(G, n, k // 2), dtype=np.uint8)
    bs = rng.integers(126, 129, size=(G, n, k // 32), dtype=np.uint8)
    buf, c = guarded((m, n), torch.float32)
    gpu_lib.mx_grouped_gemm_fp4(dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs), sizes, out=c)
    torch.cuda.synchronize()
    assert canaries_intact(buf), "mx_grouped_gemm_fp4 wrote outside C"
    want = orc.gemm_fp4_grouped(aq, as_, bq, bs, sizes)
    assert np.array_equal(to_np(c), want)


def test_grouped_gemm_fp4_mixtral_sampled(gpu_lib):
    # the Mixtral MLP's first GEMM at MXFP4: 8192 routed rows over 8 experts
    # (ragged), n = 28672, k = 4096, bf16 out; sampled rows of every expert
    rng = np.random.default_rng(78)
    sizes = [157, 574, 1914, 3333, 1056, 506, 71, 581]
    m, n, k, G = sum(sizes), 28672, 4096, len(sizes)
    aq, as_ = _fp4_operand(rng, m, k, 122, 132)
    bq = rng.integers(0, 256, size=(G, n, k // 2), dtype=np.uint8)
    bs = rng.integers(122, 133, size=(G, n, k // 32), dtype=np.uint8)
    c = gpu_lib.mx_grouped_gemm_fp4(dev_u8(aq), dev_u8(as_), dev_u8(bq), dev_u8(bs), sizes)
    torch.cuda.synchronize()
    row0 = np.concatenate([[0], np.cumsum(sizes)])
    cols = np.sort(rng.choice(n, 128, replace=False))
    for g in range(G):
        rows = np.unique(np.concatenate([[row0[g], row0[g + 1] - 1], rng.integers(row0[g], row0[g + 1], 4)]))
        got = to_np(c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
        A = orc.dequantize_rowwise_fp4(aq[rows], as_[rows])
        B = orc.dequantize_rowwise_fp4(bq[g][cols], bs[g][cols])
        want = A @ B.T
        assert np.all(np.abs(got - want) <= mfma_gemm_bound(A, B) + 2.0 ** -8 * np.abs(want)), f"expert {g}"

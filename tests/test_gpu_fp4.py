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
from tests.gpu_util import dev_bf16

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
    bits = wl.quantize_tensor_c2()
    _, _, qc, sc = gpu_lib.mx_quantize_fp4(dev_bf16(bits), colwise=True)
    torch.cuda.synchronize()
    cols = np.random.default_rng(2).choice(bits.shape[1], size=128, replace=False)
    wqc, wsc = orc.quantize_rowwise_fp4(orc.bf16_bits_to_f64(bits[:, cols]).T)
    assert np.array_equal(sc.cpu().numpy()[cols], wsc)
    assert np.array_equal(qc.cpu().numpy()[cols], wqc)

"""GPU parity of mx_quantize against the oracle: codes and scales bit-exact.

Block rule: one E8M0 scale per 32 consecutive values, E4M3 elements
("Efficient MoE training for biological foundation models", Key technical
approaches item 2), with the readings stated in the oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import canaries_intact, dev_bf16, dev_f32, guarded

pytestmark = pytest.mark.gpu


def _run(mx, x_dev, dtype, rows, cols, groups=None, row=True, col=True):
    P = sum(mx.padded_sizes(groups if groups is not None else [rows]))
    bufs = {}
    outs = {}
    if row:
        bufs["qr"], outs["qr"] = guarded((rows, cols))
        bufs["sr"], outs["sr"] = guarded((rows, cols // 32))
    if col:
        bufs["qc"], outs["qc"] = guarded((cols, P))
        bufs["sc"], outs["sc"] = guarded((cols, P // 32))
    L = mx.load()
    gs = None if groups is None else mx._i64_array(groups)
    ng = 0 if groups is None else len(groups)
    p = lambda k: mx._ptr(outs.get(k))
    st = L.mx_quantize(mx._ptr(x_dev), dtype, rows, cols, gs, ng, p("qr"), p("sr"), p("qc"), p("sc"),
                       mx._stream())
    assert st == 0, L.mx_last_error()
    torch.cuda.synchronize()
    for k, b in bufs.items():
        assert canaries_intact(b), f"out-of-bounds write around {k}"
    return {k: v.cpu().numpy() for k, v in outs.items()}


@pytest.mark.parametrize("groups", [None, [100, 0, 33, 123], [0, 256], [1], [31, 1, 32, 65]])
@pytest.mark.parametrize("cols", [32, 96, 384])
def test_quantize_bf16_groups(gpu_lib, groups, cols):
    rows = 256 if groups is None else sum(groups)
    rng = np.random.default_rng(rows * 7 + cols)
    v = (rng.standard_t(3, size=(rows, cols)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))).astype(np.float32)
    v[rng.random((rows, cols)) < 0.05] = 0.0
    v[rng.random((rows, cols)) < 0.02] *= -0.0
    bits = wl.bf16_bits_from_f32(v)
    got = _run(gpu_lib, dev_bf16(bits), 0, rows, cols, groups)
    x = orc.bf16_bits_to_f64(bits)
    qr, sr = orc.quantize_rowwise(x)
    qc, sc = orc.quantize_colwise(x, groups)
    assert np.array_equal(got["qr"], qr) and np.array_equal(got["sr"], sr)
    assert np.array_equal(got["qc"], qc) and np.array_equal(got["sc"], sc)


@pytest.mark.parametrize("shape", [(256, 64), (77, 160)])
def test_quantize_f32_input(gpu_lib, shape):
    rows, cols = shape
    rng = np.random.default_rng(rows + cols)
    v = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-140, 60, size=(rows, 1)))).astype(np.float32)
    v[0, :] = np.float32(2.0 ** -149) * rng.integers(-3, 4, size=cols)   # fp32 subnormals
    v[1, :] = -0.0
    got = _run(gpu_lib, dev_f32(v), 1, rows, cols, [rows // 2, rows - rows // 2])
    x = v.astype(np.float64)
    qr, sr = orc.quantize_rowwise(x)
    qc, sc = orc.quantize_colwise(x, [rows // 2, rows - rows // 2])
    assert np.array_equal(got["qr"], qr) and np.array_equal(got["sr"], sr)
    assert np.array_equal(got["qc"], qc) and np.array_equal(got["sc"], sc)


def test_quantize_exhaustive_bf16_times_scales(gpu_lib):
    """Every finite bf16 value in blocks whose amax is 2^(k+d), d = 0..20, as in the
    oracle's own pin: the GPU must reproduce the oracle bit for bit."""
    bits = np.arange(65536, dtype=np.uint32)
    ef = (bits >> 7) & 0xFF
    bits = bits[(ef != 0xFF) & ((bits & 0x7FFF) != 0)].astype(np.uint16)
    v = orc.bf16_bits_to_f64(bits)
    _, ex = np.frexp(np.abs(v))
    k = ex.astype(np.int64) - 1
    blocks = []
    for d in range(0, 21):
        keep = k + d <= 127                     # the anchor must itself be a finite bf16
        b = np.zeros((int(keep.sum()), 32))
        b[:, 0] = v[keep]
        b[:, 5] = np.ldexp(1.0, k[keep] + d)
        blocks.append(b)
    x = np.concatenate(blocks)                  # [n_blocks, 32]; each row is one block
    xb = wl.bf16_bits_from_f32(x.astype(np.float32))
    assert np.array_equal(orc.bf16_bits_to_f64(xb), x)
    got = _run(gpu_lib, dev_bf16(xb), 0, x.shape[0], 32, None, row=True, col=False)
    q, s = orc.quantize_rowwise(x)
    assert np.array_equal(got["sr"], s)
    assert np.array_equal(got["qr"], q)


def test_quantize_full_size_sampled(gpu_lib):
    """16384 x 4096 Student-t tensor with outliers and zero tiles, both layouts,
    in the same launch configuration the bench times; compared on 512 sampled
    rows (rowwise) and 512 sampled columns (columnwise)."""
    bits = wl.quantize_tensor_c2()
    rows, cols = bits.shape
    got = _run(gpu_lib, dev_bf16(bits), 0, rows, cols, None)
    rng = np.random.default_rng(0)
    rs = np.sort(rng.choice(rows, 512, replace=False))
    cs = np.sort(rng.choice(cols, 512, replace=False))
    # include rows/columns that cross a zeroed 32x32 tile
    x = orc.bf16_bits_to_f64(bits[rs])
    qr, sr = orc.quantize_rowwise(x)
    assert np.array_equal(got["qr"][rs], qr) and np.array_equal(got["sr"][rs], sr)
    xc = orc.bf16_bits_to_f64(bits[:, cs])
    qc, sc = orc.quantize_colwise(xc)
    assert np.array_equal(got["qc"][cs], qc) and np.array_equal(got["sc"][cs], sc)
    assert np.any(got["sr"] == 0)                # all-zero blocks exist in the data

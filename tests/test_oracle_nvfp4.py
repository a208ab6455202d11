"""Pins of the oracle's NVFP4 (reading R18: E2M1 elements, one E4M3 scale per
16 values, one float32 scale per tensor; the NVFP4 recipe of "TransformerEngine-
accelerated Llama 3 training with native PyTorch training loop", Quantized
Training, whose arithmetic the pages leave to the format's published form).

Hand-worked blocks (S = 1 because the tensor's amax is 2688 = 448 * 6):
  block [9, 4.5, 2.25, 1, 0.375, 0.75, 3.75, -9, 0 ...]:
    bmax = 9, 9 / 6 = 1.5 (exact), s = 1.5 -> E4M3 0x3C; r = 1 / 1.5 rounds to
    the float32 0.6666667; x * r in float32: 9 -> 6 (code 7), 4.5 -> 3 (5),
    2.25 -> 1.5 (3), 1 -> 0.6666667 (nearer 0.5: code 1), 0.375 -> 0.25
    exactly (a tie between 0 and 0.5: even code 0; in float64 the product is
    0.2500000075 and would give code 1), 0.75 -> 0.5 (1), 3.75 -> 2.5 exactly
    (a tie between 2 and 3: even code 4; float64 would give 5), -9 -> -6
    (code 0xF);
  block [6, -3, 1.25, 0 ...]: bmax 6, s = 1 -> 0x38, r = 1: codes 7, 0xD and
    2 (1.25 is the tie between 1 and 1.5: even code 2).
"""
import numpy as np
import pytest

import oracle as orc


def _tensor(blocks):
    """One row: a first block holding 2688 (so S = 1), then the given blocks."""
    row = [2688.0] + [0.0] * 15
    for b in blocks:
        row += list(b) + [0.0] * (16 - len(b))
    return np.array([row])


def _codes(q):
    c = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    c[:, 0::2] = q & 0xF
    c[:, 1::2] = q >> 4
    return c


def test_hand_worked_blocks():
    x = _tensor([[9, 4.5, 2.25, 1.0, 0.375, 0.75, 3.75, -9], [6, -3, 1.25]])
    q, s, amax = orc.quantize_rowwise_nvfp4(x)
    assert amax == np.float32(2688.0) and orc.nvfp4_tensor_scale(amax) == np.float32(1.0)
    assert s.tolist() == [[0x7E, 0x3C, 0x38]]                # 448, 1.5, 1.0
    c = _codes(q)[0]
    assert c[0] == 7                                         # 2688 / 448 = 6
    assert c[16:24].tolist() == [7, 5, 3, 1, 0, 1, 4, 0xF]
    assert c[32:35].tolist() == [7, 0xD, 2]
    assert not c[24:32].any() and not c[35:48].any()
    d = orc.dequantize_rowwise_nvfp4(q, s, amax)[0]
    assert d[16:24].tolist() == [9.0, 4.5, 2.25, 0.75, 0.0, 0.75, 3.0, -9.0]


def test_tensor_scale_definition():
    assert orc.nvfp4_tensor_scale(0.0) == np.float32(1.0)
    assert orc.nvfp4_tensor_scale(2688.0) == np.float32(1.0)
    assert orc.nvfp4_tensor_scale(1.0) == np.float32(2688.0)
    assert orc.nvfp4_tensor_scale(3.0) == np.float32(np.float32(2688.0) / np.float32(3.0))
    assert orc.nvfp4_tensor_scale(2.0 ** -70) == np.float32(2.0 ** 64)       # capped


def test_scaling_the_tensor_by_a_power_of_two_keeps_codes():
    """S scales by 2^-k exactly, so every float32 step of R18 sees the same
    numbers: codes and block scales are unchanged, amax scales by 2^k."""
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, size=(6, 64)) * np.exp2(rng.integers(-6, 6, size=(6, 1)))).astype(np.float32)
    q0, s0, a0 = orc.quantize_rowwise_nvfp4(x.astype(np.float64))
    for k in (-20, -3, 1, 17):
        q, s, a = orc.quantize_rowwise_nvfp4(np.ldexp(x.astype(np.float64), k))
        assert np.array_equal(q, q0) and np.array_equal(s, s0) and a == np.float32(np.ldexp(a0, k))


def test_constant_block_closed_form():
    """A tensor whose only nonzero block is 16 copies of v: S = 2688 / v,
    (v / 6) * S is 448 to within float32 rounding -> scale 0x7E; x * S / 448
    is 6 to within rounding -> code 7 (saturation absorbs the excess); the
    value decodes to 2688 / S, v to float32 precision."""
    for v in (1.0, 0.1, 3.7e-5, 1234.5):
        x = np.full((1, 16), np.float64(np.float32(v)))
        q, s, a = orc.quantize_rowwise_nvfp4(x)
        assert s.tolist() == [[0x7E]] and np.all(_codes(q) == 7)
        d = orc.dequantize_rowwise_nvfp4(q, s, a)
        assert np.allclose(d, np.float32(v), rtol=2e-7)


def test_zero_and_tiny_tensors():
    q, s, a = orc.quantize_rowwise_nvfp4(np.zeros((2, 32)))
    assert a == 0 and not q.any() and not s.any()
    # -0 keeps its sign bit (R14) in a zero-scale block
    x = np.zeros((1, 32))
    x[0, 0] = 1.0
    x[0, 17] = -1e-30                                        # (1e-30 / 6) * 2688 underflows E4M3: scale 0
    x = x.astype(np.float32).astype(np.float64)
    q, s, a = orc.quantize_rowwise_nvfp4(x)
    assert s[0, 1] == 0 and _codes(q)[0, 17] == 0x8
    # amax 2^-70: S is capped at 2^64; (2^-70 / 6) * 2^64 = 2^-6 / 6 rounds to
    # the E4M3 subnormal 2^-9 (code 1); x * 2^73 = 8 saturates to 6
    t = np.zeros((1, 16))
    t[0, 0] = 2.0 ** -70
    q, s, a = orc.quantize_rowwise_nvfp4(t)
    assert s.tolist() == [[1]] and _codes(q)[0, 0] == 7
    assert orc.dequantize_rowwise_nvfp4(q, s, a)[0, 0] == 6 * 2.0 ** -9 / 2.0 ** 64


def test_error_bound_on_random_tensors():
    """A block with a nonzero scale decodes every element to within one E2M1
    step at the top of the grid (2 units of s_b / S) plus the saturation
    excess of a rounded-down scale: |x - x^| <= 0.44 * bmax of its block. A
    block whose (bmax / 6) * S lies at or below half the smallest E4M3
    subnormal (2^-10) gets scale 0 and decodes to zeros (the spread of block
    maxima here, 20 binades, exceeds E4M3's range, so some blocks flush)."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 128)) * np.exp2(rng.integers(-10, 10, size=(8, 8)).repeat(16, axis=1)))
    x = x.astype(np.float32).astype(np.float64)
    q, s, a = orc.quantize_rowwise_nvfp4(x)
    d = orc.dequantize_rowwise_nvfp4(q, s, a)
    S = np.float64(orc.nvfp4_tensor_scale(a))
    bmax = np.abs(x).reshape(8, 8, 16).max(axis=-1)
    kept = s > 0
    assert kept.any() and (~kept).any()
    err = np.abs(d - x).reshape(8, 8, 16).max(axis=-1)
    assert np.all(err[kept] <= 0.44 * bmax[kept])
    assert np.all(d.reshape(8, 8, 16)[~kept] == 0)
    assert np.all(bmax[~kept] / 6 * S <= 2.0 ** -10 * (1 + 2.0 ** -20))
    assert np.max(err[kept] / bmax[kept]) > 0.01                          # quantization really happened


def test_colwise_is_rowwise_of_transpose_with_the_same_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((48, 32)).astype(np.float32).astype(np.float64)
    qc, sc, ac = orc.quantize_colwise_nvfp4(x)
    qr, sr, ar = orc.quantize_rowwise_nvfp4(x.T)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr) and ac == ar
    with pytest.raises(ValueError):
        orc.quantize_colwise_nvfp4(x[:40])


def _triple_loop(A, B):
    m, k = A.shape
    n = B.shape[0]
    C = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += A[i, t] * B[j, t]
            C[i, j] = acc
    return C


def test_gemm_against_brute_force_on_exact_operands():
    """Operands whose NVFP4 copies are exact: block maxima 6 with on-grid
    values and S = 1 (a 2688 in each tensor), so C is a small-integer-ish
    exact product; the GEMM must equal a brute-force triple loop of the
    inputs themselves."""
    rng = np.random.default_rng(2)
    grid = orc.E2M1_VALUES
    def operand(rows, k):
        v = rng.choice(grid, size=(rows, k)) * rng.choice([-1, 1], size=(rows, k))
        v[:, ::16] = 6.0                                     # every block's max is 6: scale 1
        v[0, 0] = 2688.0                                     # amax 2688: S = 1 (block 0 of row 0 scale 448)
        v[0, 1:16] = 0.0
        return v
    A, B = operand(5, 64), operand(7, 64)
    aq, as_, aa = orc.quantize_rowwise_nvfp4(A)
    bq, bs, ba = orc.quantize_rowwise_nvfp4(B)
    assert np.array_equal(orc.dequantize_rowwise_nvfp4(aq, as_, aa), A)
    assert np.array_equal(orc.gemm_nvfp4(aq, as_, aa, bq, bs, ba), _triple_loop(A, B))


def test_grouped_gemm_is_loop_of_dense_with_per_group_scales():
    rng = np.random.default_rng(4)
    sizes = [3, 0, 5]
    A = rng.standard_normal((8, 32)).astype(np.float32).astype(np.float64)
    aq, as_, aa = orc.quantize_rowwise_nvfp4(A)
    Bs = [(rng.standard_normal((6, 32)) * 10.0 ** g).astype(np.float32).astype(np.float64) for g in range(3)]
    bqs = [orc.quantize_rowwise_nvfp4(b) for b in Bs]
    bq = np.stack([b[0] for b in bqs])
    bs = np.stack([b[1] for b in bqs])
    ba = np.array([b[2] for b in bqs], dtype=np.float32)
    C = orc.gemm_nvfp4_grouped(aq, as_, aa, bq, bs, ba, sizes)
    assert np.allclose(C[:3], orc.gemm_nvfp4(aq[:3], as_[:3], aa, bq[0], bs[0], ba[0]), rtol=0, atol=0)
    assert np.allclose(C[3:], orc.gemm_nvfp4(aq[3:], as_[3:], aa, bq[2], bs[2], ba[2]), rtol=0, atol=0)
    assert ba[0] != ba[2]                                    # the groups really carry different tensor scales


def test_rejects_bad_shapes_and_values():
    with pytest.raises(ValueError):
        orc.quantize_rowwise_nvfp4(np.zeros((2, 24)))
    with pytest.raises(ValueError):
        orc.quantize_rowwise_nvfp4(np.full((1, 16), np.inf))
    with pytest.raises(ValueError):
        orc.quantize_rowwise_nvfp4(np.full((1, 16), 0.1))    # not an exact float32

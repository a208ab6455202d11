"""Pins of the oracle's MXFP4 columnwise layout and weight-gradient product
(reading R16: per-group padding of R6 with R14's elements; the group-K
product of R15 per group)."""
import numpy as np

import oracle as orc


def _codes(q):
    c = np.empty((q.shape[0], 2 * q.shape[1]), dtype=np.uint8)
    c[:, 0::2], c[:, 1::2] = q & 0xF, q >> 4
    return c


def test_colwise_layout_exact_on_grid_values():
    # every value is +-1, 2 or 4: with amax 4 the block scale is 2^0 (code 127)
    # and each value is an E2M1 grid point, so the layout is read back exactly
    sizes = [5, 0, 40, 32]
    R, C = sum(sizes), 64
    r = np.arange(R)[:, None]
    c = np.arange(C)[None, :]
    x = np.exp2(((r + 2 * c) % 3).astype(np.float64)) * np.where((r * 7 + c) % 5 == 0, -1.0, 1.0)
    x[np.arange(R) % 7 == 3] = 4.0            # every 32-row block has amax 4
    q, s = orc.quantize_colwise_fp4(x, sizes)
    P = orc.padded_sizes(sizes).tolist()
    assert P == [32, 0, 64, 32] and q.shape == (C, 64) and s.shape == (C, 4)
    deq = orc.dequantize_rowwise_fp4(q, s)
    r0, p0 = 0, 0
    for m, p in zip(sizes, P):
        np.testing.assert_array_equal(deq[:, p0:p0 + m], x[r0:r0 + m].T)
        assert np.all(deq[:, p0 + m:p0 + p] == 0)           # padding rows are zeros
        assert np.all(_codes(q)[:, p0 + m:p0 + p] == 0)
        r0 += m
        p0 += p
    # a block that holds only the padding of the 5-row group still has amax 4 (rows 3 is 4)
    assert np.all(s[:, 0] == 127)


def test_colwise_matches_rowwise_of_transpose_for_one_group():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((96, 64)) * np.exp2(rng.integers(-6, 6, size=(96, 1)))
    q, s = orc.quantize_colwise_fp4(x)
    qt, st = orc.quantize_rowwise_fp4(x.T)
    np.testing.assert_array_equal(q, qt)
    np.testing.assert_array_equal(s, st)


def test_group_k_per_group_constants():
    # A and B constant within each group's rows: C_g = m_g * a_g * b_g exactly
    sizes = [7, 0, 33, 64]
    M, N = 64, 96
    vals_a, vals_b = [1.5, 3.0, -2.0, 0.5], [4.0, 6.0, 1.0, -3.0]
    xa = np.concatenate([np.full((m, M), v) for m, v in zip(sizes, vals_a)])
    xb = np.concatenate([np.full((m, N), v) for m, v in zip(sizes, vals_b)])
    aq, as_ = orc.quantize_colwise_fp4(xa, sizes)
    bq, bs = orc.quantize_colwise_fp4(xb, sizes)
    C = orc.gemm_fp4_group_k(aq, as_, bq, bs, sizes)
    assert C.shape == (4, M, N)
    for g, m in enumerate(sizes):
        np.testing.assert_array_equal(C[g], np.full((M, N), m * vals_a[g] * vals_b[g]))


def test_group_k_brute_force():
    rng = np.random.default_rng(5)
    sizes = [3, 40, 0, 9]
    M, N = 5, 4
    K = int(orc.padded_sizes(sizes).sum())
    aq = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    as_ = rng.integers(120, 135, size=(M, K // 32), dtype=np.uint8)
    bs = rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8)
    C = orc.gemm_fp4_group_k(aq, as_, bq, bs, sizes)
    ca, cb = _codes(aq), _codes(bq)
    k0 = 0
    for g, p in enumerate(orc.padded_sizes(sizes).tolist()):
        for i in range(M):
            for j in range(N):
                acc = 0.0
                for k in range(k0, k0 + p):
                    va = float(orc.e2m1_value(ca[i, k])) * 2.0 ** (int(as_[i, k // 32]) - 127)
                    vb = float(orc.e2m1_value(cb[j, k])) * 2.0 ** (int(bs[j, k // 32]) - 127)
                    acc += va * vb
                assert C[g, i, j] == acc
        k0 += p

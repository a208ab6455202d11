"""Pins of the oracle's MXFP4 quantizer (reading R14): the E2M1 value table,
a hand-worked block with every tie of the grid, an arithmetic second
formulation of the encoder over many values, scale equivariance, round trip
and the zero block."""
import numpy as np

import oracle as orc


def test_e2m1_table():
    assert orc.e2m1_value(np.arange(8)).tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert orc.e2m1_value(np.arange(8, 16)).tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_hand_worked_block():
    # amax 7 -> floor(log2 7) = 2 -> e = 0 -> scale code 127; t = v
    v = np.zeros(32)
    v[:12] = [0.1, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, -0.3, -1.1]
    # nearest, ties to the even code: 0.25 -> 0, 0.75 -> 1.0 (code 2), 1.25 -> 1.0,
    # 1.75 -> 2.0 (code 4), 2.5 -> 2.0, 3.5 -> 4.0 (code 6), 5 -> 4.0, 6 -> 6,
    # 7 saturates to 6; -0.3 -> -0.5 (code 9), -1.1 -> -1.0 (code 10)
    want = [0, 0, 2, 2, 4, 4, 6, 6, 7, 7, 9, 10] + [0] * 20
    q, s = orc.quantize_rowwise_fp4(v[None, :])
    assert s.tolist() == [[127]]
    codes = np.empty(32, dtype=np.uint8)
    codes[0::2], codes[1::2] = q[0] & 0xF, q[0] >> 4
    assert codes.tolist() == want
    assert q[0, 0] == 0x00 and q[0, 1] == 0x22 and q[0, 4] == 0x77


def _arith_encode(t):
    """Second formulation: scale |t| onto the grid of its binade and round
    half to even on the integer grid index."""
    a = np.abs(t)
    out = np.empty(a.shape, dtype=np.int64)
    for i, x in np.ndenumerate(a):
        if x >= 6.0:
            c = 7
        elif x < 1.0:
            c = int(np.rint(x * 2.0))                  # grid 0, 0.5, 1 -> codes 0, 1, 2
        else:
            E = int(np.floor(np.log2(x)))              # 0, 1 or 2 (x < 6)
            m = np.rint((x / 2.0 ** E - 1.0) * 2.0)    # 0, 1 or 2 (carry)
            c = 2 * (E + 1) + int(m)
            c = min(c, 7)
        out[i] = c | (8 if np.signbit(t[i]) else 0)
    return out


def test_encoder_matches_arithmetic_formulation():
    rng = np.random.default_rng(80)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    t = np.concatenate([rng.uniform(-8, 8, 4000), ties, -ties, np.linspace(0, 7, 281), [-0.0, 6.0, 6.5]])
    assert np.array_equal(orc.e2m1_encode(t).astype(np.int64), _arith_encode(t))


def test_scale_equivariance_round_trip_and_zero():
    rng = np.random.default_rng(81)
    x = rng.standard_normal((6, 64))
    q, s = orc.quantize_rowwise_fp4(x)
    q2, s2 = orc.quantize_rowwise_fp4(x * 2.0 ** 5)
    assert np.array_equal(q, q2) and np.array_equal(s2, s + 5)
    # the block amax lands in [4, 8) / 2^e, so its code is 6 (4.0) or 7 (6.0);
    # dequantized values quantize back to the same codes and scales
    xd = orc.dequantize_rowwise_fp4(q, s)
    q3, s3 = orc.quantize_rowwise_fp4(xd)
    assert np.array_equal(q3, q) and np.array_equal(s3, s)
    qz, sz = orc.quantize_rowwise_fp4(np.zeros((1, 32)))
    assert qz.tolist() == [[0] * 16] and sz.tolist() == [[0]]


# ---- the MXFP4 GEMM of the oracle (gemm_fp4): closed forms

def _fill(rows, k, code, scale):
    """rows x k operand whose every element has E2M1 code `code` (per row) and
    every block scale code `scale` (per row)."""
    code = np.asarray(code, dtype=np.uint8).reshape(-1, 1)
    q = np.repeat(code | (code << 4), k // 2, axis=1).astype(np.uint8)
    s = np.repeat(np.asarray(scale, dtype=np.uint8).reshape(-1, 1), k // 32, axis=1)
    return q, s


def test_gemm_fp4_constant_rows():
    # row i of A is the constant v_i, row j of B is w_j: C[i, j] = k v_i w_j.
    # m != n, so a transposed operand or output changes the shape or values.
    k = 128
    a_codes, a_vals = [2, 7, 10, 5], [1.0, 6.0, -1.0, 3.0]          # 1, 6, -1, 3
    b_codes, b_vals = [1, 12, 3], [0.5, -2.0, 1.5]
    aq, as_ = _fill(4, k, a_codes, [127, 128, 126, 127])            # scales 1, 2, 1/2, 1
    bq, bs = _fill(3, k, b_codes, [127, 127, 129])                  # scales 1, 1, 4
    C = orc.gemm_fp4(aq, as_, bq, bs)
    av = np.array(a_vals) * np.array([1.0, 2.0, 0.5, 1.0])
    bv = np.array(b_vals) * np.array([1.0, 1.0, 4.0])
    assert C.shape == (4, 3)
    assert np.array_equal(C, k * np.outer(av, bv))


def test_gemm_fp4_single_nonzero_element():
    # one nonzero element per operand row at chosen k: C[i, j] is their product
    # when the positions match and 0 otherwise; checks the nibble -> k order
    # (element 2i in the low nibble) and the block -> scale pairing
    k = 64
    aq = np.zeros((2, k // 2), dtype=np.uint8)
    bq = np.zeros((2, k // 2), dtype=np.uint8)
    as_ = np.full((2, 2), 127, dtype=np.uint8)
    bs = np.full((2, 2), 127, dtype=np.uint8)
    aq[0, 20] = 0x07         # A[0, 40] = 6 (low nibble = even element 40), block 1
    aq[1, 20] = 0x70         # A[1, 41] = 6 (high nibble = odd element 41)
    bq[0, 20] = 0x05         # B[0, 40] = 3
    bq[1, 20] = 0x30         # B[1, 41] = 1.5
    as_[0, 1] = 129          # block 1 of A row 0 scaled by 4
    bs[1, 0] = 140           # block 0 of B row 1: no nonzero element there
    C = orc.gemm_fp4(aq, as_, bq, bs)
    assert C.tolist() == [[6 * 4 * 3, 0.0], [0.0, 6 * 1.5]]


def test_gemm_fp4_matches_blockwise_sum():
    # C equals the sum over 32-blocks of 2^(sa + sb) times the integer-grid
    # dot product of the block's E2M1 values (values doubled to integers)
    rng = np.random.default_rng(7)
    m, n, k = 5, 6, 128
    aq = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    as_ = rng.integers(120, 135, size=(m, k // 32), dtype=np.uint8)
    bs = rng.integers(120, 135, size=(n, k // 32), dtype=np.uint8)
    twice = {c: int(round(2 * v)) for c, v in enumerate(orc.E2M1_VALUES)}   # 0..12

    def ints(q):
        out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.int64)
        for r in range(q.shape[0]):
            for j in range(q.shape[1]):
                for half, c in enumerate((int(q[r, j]) & 0xF, int(q[r, j]) >> 4)):
                    v = twice[c & 7]
                    out[r, 2 * j + half] = -v if c & 8 else v
        return out

    ai, bi = ints(aq), ints(bq)
    want = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            for b in range(k // 32):
                dot = int(np.dot(ai[i, 32 * b:32 * b + 32], bi[j, 32 * b:32 * b + 32]))
                want[i, j] += dot * 2.0 ** (int(as_[i, b]) + int(bs[j, b]) - 254 - 2)
    assert np.array_equal(orc.gemm_fp4(aq, as_, bq, bs), want)


def test_gemm_fp4_grouped_reduces_to_dense_and_routes_rows():
    # groups of one shared weight equal the dense GEMM; with per-group
    # constant weights w_g each output row carries its own group's w_g, so a
    # row credited to the wrong group (or an empty group taking rows) fails
    rng = np.random.default_rng(11)
    sizes = [3, 0, 5, 1, 0]
    m, n, k = sum(sizes), 4, 64
    aq = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    as_ = rng.integers(124, 131, size=(m, k // 32), dtype=np.uint8)
    bq1 = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    bs1 = rng.integers(124, 131, size=(n, k // 32), dtype=np.uint8)
    G = len(sizes)
    same = orc.gemm_fp4_grouped(aq, as_, np.stack([bq1] * G), np.stack([bs1] * G), sizes)
    assert np.array_equal(same, orc.gemm_fp4(aq, as_, bq1, bs1))
    # B_g all ones times 2^g: C[r, j] = 2^g(r) * sum_k A[r, k]
    bq = np.full((G, n, k // 2), 0x22, dtype=np.uint8)
    bs = np.stack([np.full((n, k // 32), 127 + g, dtype=np.uint8) for g in range(G)])
    C = orc.gemm_fp4_grouped(aq, as_, bq, bs, sizes)
    rowsum = orc.dequantize_rowwise_fp4(aq, as_).sum(axis=1)
    owner = np.repeat(np.arange(G), sizes)
    assert np.array_equal(C, (rowsum * 2.0 ** owner)[:, None] * np.ones((1, n)))

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

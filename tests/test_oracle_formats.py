"""Pins of the oracle's number formats and block quantizer against facts that do
not come from the oracle itself: closed-form anchors of E4M3/E8M0, brute-force
nearest-value search, hand-worked blocks (tests/golden/mx_blocks.txt) and
invariants of the block-scaling definition (one E8M0 scale per 32 consecutive
values, E4M3 elements: "Efficient MoE training for biological foundation
models", Key technical approaches item 2)."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")


# ---------------------------------------------------------------------------
# closed-form anchors

def test_e4m3_anchor_values():
    v = orc.e4m3_value(np.arange(256, dtype=np.uint8))
    assert v[0x7E] == 448.0                    # largest normal 1.75 * 2^8
    assert v[0x08] == 2.0 ** -6                # smallest normal
    assert v[0x01] == 2.0 ** -9                # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9            # largest subnormal
    assert v[0x38] == 1.0                      # exponent field 7 = bias
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0xFE] == -448.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)            # codes 0..0x7E strictly increasing
    assert np.array_equal(v[0x80:0xFF], -pos)  # sign-magnitude
    assert np.count_nonzero(np.isnan(v)) == 2  # no infinities, two NaNs


def test_e8m0_anchor_values():
    s = orc.e8m0_value(np.arange(256))
    assert s[127] == 1.0 and s[0] == 2.0 ** -127 and s[254] == 2.0 ** 127
    assert np.isnan(s[255])


# ---------------------------------------------------------------------------
# encode vs brute-force nearest search

_POS = orc.e4m3_value(np.arange(0x7F, dtype=np.uint8))   # the 127 finite magnitudes


def _brute_code(t):
    """Nearest finite E4M3 magnitude (ties -> even code), sign from t.  Values
    beyond 448 are nearest to 448, so saturation needs no separate rule."""
    t = np.asarray(t, dtype=np.float64)
    d = np.abs(np.abs(t)[:, None] - _POS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(0x7F)
    # among tied candidates (at most two) take the even code
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return (pick | np.where(np.signbit(t), 0x80, 0)).astype(np.uint8)


def _all_bf16_magnitudes_scaled(kmin=-16, kmax=10):
    m = 1.0 + np.arange(128) / 128.0
    vals = [m * 2.0 ** k for k in range(kmin, kmax)]
    return np.concatenate(vals)


def test_encode_matches_brute_force_on_bf16_grid():
    t = _all_bf16_magnitudes_scaled()
    t = np.concatenate([t, -t, [0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e9]])
    assert np.array_equal(orc.e4m3_encode(t), _brute_code(t))


def test_encode_matches_brute_force_on_all_midpoints():
    pos = _POS
    mids = (pos[:-1] + pos[1:]) / 2.0            # exact halfway points: ties
    t = np.concatenate([mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e3)])
    assert np.array_equal(orc.e4m3_encode(t), _brute_code(t))


def test_encode_matches_brute_force_random_fp32():
    rng = np.random.default_rng(0)
    t = (rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 10, 200000))).astype(np.float32)
    t = t.astype(np.float64)
    assert np.array_equal(orc.e4m3_encode(t), _brute_code(t))


def _bf16_exponent(bits):
    """floor(log2 |v|) of a finite nonzero bf16 from its bit pattern."""
    ef = (bits >> 7) & 0xFF
    mant = bits & 0x7F
    out = ef.astype(np.int64) - 127
    sub = ef == 0
    # subnormal: value = mant * 2^-133; floor(log2) = bit_length(mant) - 1 - 133
    bl = np.array([int(m).bit_length() for m in mant[sub]], dtype=np.int64)
    out[sub] = bl - 1 - 133
    return out


def test_quantize_exhaustive_bf16_times_scales():
    """Every finite bf16 value, in blocks whose amax is a power of two 2^(k+d)
    (k = the value's own binary exponent, d = 0..20): the scale follows from the
    construction and the code from the brute-force search."""
    bits = np.arange(65536, dtype=np.uint32)
    ef = (bits >> 7) & 0xFF
    bits = bits[(ef != 0xFF) & ((bits & 0x7FFF) != 0)].astype(np.uint16)
    v = orc.bf16_bits_to_f64(bits)
    k = _bf16_exponent(bits.astype(np.int64))
    for d in range(0, 21):
        anchor = np.ldexp(1.0, k + d)
        blocks = np.zeros((len(v), 32))
        blocks[:, 0] = v
        blocks[:, 1] = anchor
        codes, scales = orc.quantize_blocks(blocks)
        e = np.clip(k + d - 8, -127, 127)
        assert np.array_equal(scales, (e + 127).astype(np.uint8)), d
        exp0 = _brute_code(np.ldexp(v, -e))
        assert np.array_equal(codes[:, 0], exp0), d
        assert np.array_equal(codes[:, 1], _brute_code(np.ldexp(anchor, -e))), d
        assert np.all(codes[:, 2:] == 0)


# ---------------------------------------------------------------------------
# hand-worked blocks

def _parse_value(tok):
    rep = 1
    if "x" in tok.split("^")[-1]:
        tok, r = tok.rsplit("x", 1)
        rep = int(r)
    p, k = tok.split("*2^")
    neg = p.startswith("-")
    val = Fraction(int(p)) * (Fraction(2) ** int(k))
    f = float(val)
    if neg and val == 0:
        f = -0.0
    return [f] * rep


def _golden_blocks():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, vals, scale, codes = [s.strip() for s in line.split("|")]
        v = []
        for tok in vals.split():
            v += _parse_value(tok)
        assert len(v) == 32, name
        c = [int(h, 16) for h in codes.split()]
        assert len(c) == 32, name
        out.append((name, np.array(v), int(scale, 16), np.array(c, dtype=np.uint8)))
    return out


@pytest.mark.parametrize("blk", _golden_blocks(), ids=lambda b: b[0])
def test_hand_worked_block(blk):
    name, v, scale, codes = blk
    q, s = orc.quantize_blocks(v[None, :])
    assert int(s[0]) == scale
    assert np.array_equal(q[0], codes)


# ---------------------------------------------------------------------------
# invariants

def _random_blocks(n=20000, seed=1):
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-30, 30, size=(n, 1)))
    v = (rng.standard_t(3, size=(n, 32)) * mag).astype(np.float32).astype(np.float64)
    return v


def test_round_trip_of_codes():
    """Codes whose largest magnitude lies in [0x78, 0x7E] re-quantize to themselves."""
    rng = np.random.default_rng(2)
    c = rng.integers(0, 0x7F, size=(5000, 32)).astype(np.uint8)
    c[:, 0] = rng.integers(0x78, 0x7F, size=5000)
    c = c | (rng.integers(0, 2, size=c.shape).astype(np.uint8) << 7)
    s = rng.integers(20, 230, size=5000).astype(np.uint8)
    v = orc.e4m3_value(c) * orc.e8m0_value(s)[:, None]
    q2, s2 = orc.quantize_blocks(v)
    # -0 and +0 both decode to 0; compare magnitudes for zero codes, else exact
    zero = (c & 0x7F) == 0
    assert np.array_equal(s2, s)
    assert np.array_equal(np.where(zero, 0, q2), np.where(zero, 0, c))


def test_scale_equivariance():
    v = _random_blocks()
    q, s = orc.quantize_blocks(v)
    for k in (-7, 1, 5):
        q2, s2 = orc.quantize_blocks(np.ldexp(v, k))
        ok = (s.astype(int) + k >= 0) & (s.astype(int) + k <= 254) & (s > 0)
        assert np.array_equal(q2[ok], q[ok])
        assert np.array_equal(s2[ok].astype(int), s[ok].astype(int) + k)


def test_amax_code_range_and_error_bound():
    v = _random_blocks()
    q, s = orc.quantize_blocks(v)
    i = np.argmax(np.abs(v), axis=1)
    top = q[np.arange(len(v)), i] & 0x7F
    assert np.all((top >= 0x78) & (top <= 0x7E))
    X = orc.e8m0_value(s)[:, None]
    vh = orc.e4m3_value(q) * X
    t = np.abs(v) / X
    err = np.abs(vh - v)
    normal = (t >= 2.0 ** -6) & (t < 448)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v[normal]))
    sub = t < 2.0 ** -6
    assert np.all(err[sub] <= (2.0 ** -10) * np.broadcast_to(X, v.shape)[sub])
    sat = t >= 448
    assert np.all(np.abs(vh[sat]) == 448.0 * np.broadcast_to(X, v.shape)[sat])


def test_sign_and_monotone():
    v = _random_blocks(5000)
    q, s = orc.quantize_blocks(v)
    assert np.array_equal((q >> 7) == 1, np.signbit(v))
    vh = orc.e4m3_value(q)
    for r in range(0, 5000, 97):
        o = np.argsort(v[r], kind="stable")
        assert np.all(np.diff(vh[r][o]) >= 0)


def test_zero_blocks():
    q, s = orc.quantize_blocks(np.zeros((3, 32)))
    assert np.all(q == 0) and np.all(s == 0)


def test_nonfinite_rejected():
    with pytest.raises(ValueError):
        orc.quantize_blocks(np.full((1, 32), np.inf))


def test_colwise_is_rowwise_of_transpose():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((96, 64)).astype(np.float32).astype(np.float64)
    qc, sc = orc.quantize_colwise(x)
    qr, sr = orc.quantize_rowwise(x.T)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)


def test_grouped_colwise_is_padded_per_group_transpose():
    rng = np.random.default_rng(4)
    sizes = [17, 0, 32, 45]
    x = rng.standard_normal((sum(sizes), 64)) * 3
    q, s = orc.quantize_colwise(x, sizes)
    assert q.shape == (64, 32 + 0 + 32 + 64)
    r0, c0 = 0, 0
    for m in sizes:
        p = -(-m // 32) * 32
        if p:
            pad = np.zeros((p, 64))
            pad[:m] = x[r0:r0 + m]
            qr, sr = orc.quantize_rowwise(pad.T)
            assert np.array_equal(q[:, c0:c0 + p], qr)
            assert np.array_equal(s[:, c0 // 32:(c0 + p) // 32], sr)
            assert np.all(q[:, c0 + m:c0 + p] == 0)
        r0 += m
        c0 += p


# ---------------------------------------------------------------------------
# bf16 rounding vs nearest search over the whole bf16 grid

def test_round_to_bf16_vs_grid_search():
    bits = np.arange(0x7F80, dtype=np.uint16)                 # +0 .. largest finite
    grid = orc.bf16_bits_to_f64(bits)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(50000) * np.exp2(rng.uniform(-135, 120, 50000))
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([x, mids[::97], -mids[::89]])
    a = np.abs(x)
    j = np.clip(np.searchsorted(grid, a), 1, len(grid) - 1)
    lo, hi = grid[j - 1], grid[j]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & (bits[j] % 2 == 0))
    want = np.copysign(np.where(pick_hi, hi, lo), x)
    assert np.array_equal(orc.round_to_bf16(x), want)

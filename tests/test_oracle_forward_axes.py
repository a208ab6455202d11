"""Pins of the copies the oracle's forward GEMMs read, in both block formats
(readings R8, R17): H1 = rowwise(X) . rowwise(W1)^T and Y = rowwise(A) .
rowwise(W2)^T, every block running along its GEMM's contraction axis, and A
requantized after it is formed.

Source: "Efficient MoE training for biological foundation models", Key
technical approaches item 3 (GroupedLinear -> ScaledSwiGLU -> GroupedLinear
on MXFP8 copies); the MXFP4 form is reading R17.

Constructions (worked by hand):
  * X and W1 -- s and 1 share a 32-block along H, s is alone along the other
    axis; the picked H1 entry equals that operand's element, so it is Q when
    the block runs along H and s otherwise (s, Q as in the backward pins:
    MXFP8 s = 9 * 2^-19, Q = 2^-16; MXFP4 s = 1.5 * 2^-4, Q = 2^-3).
  * A and W2 -- A is a transcendental function of H1, so these pins use a
    flush instead: an element 2^-20 times smaller than the largest in its
    block quantizes to 0 in either format (MXFP8: at most 2^-20 * 2^9 below
    the E4M3 grid's first step, 2^-9 of the scaled unit; MXFP4: at most
    2^-20 * 2^3 < 0.25), while alone in its block it is kept (to within one
    rounding of itself). With gate g = 1 in both columns, up = (2^-20, 1) makes
    A[0] = (2^-20 * c, c) with c = silu(1): rowwise, A[0, 0] is flushed;
    columnwise (alone in column 0) it is not. W2 row 0 = (2^-20, 1) with A's
    column 1 zero does the same for W2.
"""
import numpy as np
import pytest

import oracle as orc
from oracle import mx_oracle as mxo

FORMATS = {
    "mxfp8": (True, 9.0 * 2.0 ** -19, 2.0 ** -16),
    "mxfp4": ("mxfp4", 1.5 * 2.0 ** -4, 2.0 ** -3),
}
H, F, R = 64, 64, 40
TINY = 2.0 ** -20


def _base():
    return dict(x=np.zeros((R, H)), w1=np.zeros((1, 2 * F, H)), w2=np.zeros((1, H, F)),
                probs=np.ones(R))


def _run(c, quantize):
    return orc.mlp_forward(c["x"], c["probs"], c["w1"], c["w2"], [R], quantize=quantize)


def pin_x_rowwise(S, Q):
    """X row 0 = (s, 1, 0...) along H; column 0 of X holds s alone. Up row 0
    of W1 is e_0, so u[0, 0] = Xq[0, 0]."""
    c = _base()
    c["x"][0, 0] = S
    c["x"][0, 1] = 1.0
    c["w1"][0, F + 0, 0] = 1.0
    return c, lambda f: f["h1"][0, F] == Q


def pin_w1_rowwise(S, Q):
    """Up row 0 of W1 = (s, 1, 0...) along H; column 0 of W1 holds s alone
    (the other rows are 0). X row 0 = e_0, so u[0, 0] = W1q[F, 0]."""
    c = _base()
    c["w1"][0, F + 0, 0] = S
    c["w1"][0, F + 0, 1] = 1.0
    c["x"][0, 0] = 1.0
    return c, lambda f: f["h1"][0, F] == Q


def pin_a_rowwise(S, Q):
    """X row 0 = e_0; gate rows 0 and 1 of W1 take h = 0 with weight 1 (g = 1),
    up rows 0 and 1 weights TINY and 1. A[0] = (TINY c, c, 0...), column 0 of
    A holds TINY c alone. W2[0, 0] = 1 picks Aq[0, 0]: 0 when A is quantized
    along F."""
    c = _base()
    c["x"][0, 0] = 1.0
    c["w1"][0, 0, 0] = 1.0
    c["w1"][0, 1, 0] = 1.0
    c["w1"][0, F + 0, 0] = TINY
    c["w1"][0, F + 1, 0] = 1.0
    c["w2"][0, 0, 0] = 1.0
    return c, lambda f: f["y_exact"][0, 0] == 0.0 and f["a"][0, 0] != 0.0


def pin_w2_rowwise(S, Q):
    """W2 row 0 = (TINY, 1, 0...) along F, column 0 of W2 holds TINY alone; A
    row 0 = (c, 0, ...) (gate 1, up 1 in column 0 only). Y[0, 0] = Aq[0, 0] *
    W2q[0, 0]: 0 when W2 is quantized along F."""
    c = _base()
    c["x"][0, 0] = 1.0
    c["w1"][0, 0, 0] = 1.0
    c["w1"][0, F + 0, 0] = 1.0
    c["w2"][0, 0, 0] = TINY
    c["w2"][0, 0, 1] = 1.0
    return c, lambda f: f["y_exact"][0, 0] == 0.0 and f["a"][0, 0] != 0.0


PINS = [pin_x_rowwise, pin_w1_rowwise, pin_a_rowwise, pin_w2_rowwise]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_forward_operand_axis(pin, fmt):
    quantize, S, Q = FORMATS[fmt]
    c, ok = pin(S, Q)
    assert ok(_run(c, quantize)), pin.__name__


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_flush_values(fmt):
    """The flush the A and W2 pins rely on, and that the element is kept when
    alone in its block, from the encoders themselves."""
    quantize = FORMATS[fmt][0]
    c = 1.0 * orc.sigmoid(1.0)
    row = np.zeros((1, 32))
    row[0, 0], row[0, 1] = TINY * c, c
    assert mxo._qdq_row(row, quantize)[0, 0] == 0.0
    alone = np.zeros((1, 32))
    alone[0, 0] = TINY * c
    assert abs(mxo._qdq_row(alone, quantize)[0, 0] / (TINY * c) - 1) < 0.25


def test_formats_differ_on_the_pins():
    """MXFP8 keeps the MXFP4 pin value s = 1.5 * 2^-4 exact next to 1 (24 *
    2^-8 is an E4M3 value at scale 2^-8), so a forward that quantized with
    the wrong format fails the MXFP4 pins."""
    _, S4, Q4 = FORMATS["mxfp4"]
    c, ok = pin_x_rowwise(S4, Q4)
    assert ok(_run(c, "mxfp4"))
    assert not ok(_run(c, True))


# Call sites of the quantize-dequantize helper in mlp_forward, in evaluation
# order for one expert: X (once, before the expert loop), W1, W2, A.
FWD_SITES = 4


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("site", range(FWD_SITES))
def test_each_swapped_forward_axis_fails_a_pin(monkeypatch, site, fmt):
    """A planted mistake (CPU only): call `site` quantizes along the other
    axis; some pin must fail."""
    quantize, S, Q = FORMATS[fmt]
    row, col = mxo._qdq_row, mxo._qdq_col
    count = {"n": 0}

    def f(x, q):
        i = count["n"] % FWD_SITES
        count["n"] += 1
        return (col if i == site else row)(x, q)

    monkeypatch.setattr(mxo, "_qdq_row", f)
    caught = []
    for pin in PINS:
        count["n"] = 0
        c, ok = pin(S, Q)
        if not ok(_run(c, quantize)):
            caught.append(pin.__name__)
    assert caught, f"swapping the axis of forward call site {site} passes every pin"

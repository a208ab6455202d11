"""Pins of which MXFP8 (and, reading R17, MXFP4) copy each straight-through
backward GEMM of the oracle reads (reading R9): dA = rowwise(dY) . columnwise(W2), dX = rowwise(dH1) .
columnwise(W1), dW2 = columnwise(dY)^T . columnwise(A), dW1 = columnwise(dH1)^T
. columnwise(X), the columnwise blocks of activations and gradients
restarting at each expert's first row.

Source: "Efficient MoE training for biological foundation models", Key
technical approaches item 3 (a fused forward op and a corresponding fused
backward op, MXFP8 on both); the copy each GEMM takes is the one whose 32-value
blocks run along that GEMM's contraction axis, since a block scale can only be
factored out of a dot product along the block.

Construction (values worked by hand). s = 9 * 2^-19 = 1.125 * 2^-16 is an
exact E4M3 value at its own scale (floor(log2 s) = -16, e = -24, s / 2^e =
288 = 1.125 * 2^8). In a 32-block whose largest magnitude is 1 (e = -8), s /
2^e = 9 * 2^-11 lies on the E4M3 subnormal grid of step 2^-9 at 2.25 steps,
so it rounds to 2 steps: s quantizes to Q = 2^-16 there. Each pin puts s and
1 in the same block along one axis of one operand and s alone along the
other axis, and makes the GEMM output equal that operand element times 1, so
the output is Q when the operand is quantized along the expected axis and s
when along the other one.

MXFP4 (R14): s = 1.5 * 2^-4 is exact at its own scale (floor(log2 s) = -4,
e = -6, s / 2^e = 6, E2M1's largest value). In a 32-block whose largest
magnitude is 1 (e = -2), s / 2^e = 0.375 lies between the E2M1 values 0 and
0.5, nearer 0.5, so s quantizes to Q = 0.5 * 2^-2 = 2^-3 there. 1, 2 and 2s
are exact in either format, so the same constructions pin both.

The backward is driven through a hand-made forward record (H1 = [g | u] and
A): with g = 0, sigmoid(0) = 1/2 and silu(0) = 0, so the SwiGLU backward
gives exactly dg = dA * w * u / 2 and du = 0.
"""
import numpy as np
import pytest

import oracle as orc
from oracle import mx_oracle as mxo

# format -> (quantize argument of the oracle, s exact at its own scale, Q = s
# quantized inside a block whose amax is 1)
FORMATS = {
    "mxfp8": (True, 9.0 * 2.0 ** -19, 2.0 ** -16),
    "mxfp4": ("mxfp4", 1.5 * 2.0 ** -4, 2.0 ** -3),
}
H, F, R = 64, 64, 40


def _base(split=(R,)):
    """All-zero inputs of one MLP: x [R,H], w1 [E,2F,H], w2 [E,H,F], dy [R,H],
    forward record with H1 = 0 and A = 0, routing weights 1."""
    E = len(split)
    rows = int(sum(split))
    return dict(x=np.zeros((rows, H)), w1=np.zeros((E, 2 * F, H)), w2=np.zeros((E, H, F)),
                dy=np.zeros((rows, H)), h1=np.zeros((rows, 2 * F)), a=np.zeros((rows, F)),
                probs=np.ones(rows), split=list(split))


def _unit_da(c):
    """dA = 1 everywhere: dY[:, 0] = 1 and row 0 of W2 all ones (both exact in
    either layout)."""
    c["dy"][:, 0] = 1.0
    c["w2"][:, 0, :] = 1.0


def _run(c, quantize):
    fwd = dict(h1_bf16=c["h1"], h1=c["h1"], a=c["a"])
    return orc.mlp_backward(c["x"], c["probs"], c["w1"], c["w2"], c["split"], c["dy"], fwd,
                            quantize=quantize)


# -- each pin: (inputs, extractor of the pinned output) ------------------------

def pin_da_w2_columnwise(S):
    """dA = dY . W2 (K = H): W2 column 0 holds s (h=0) and 1 (h=1) in one
    block along H; row h=0 of W2 holds s alone along F."""
    c = _base()
    c["dy"][:, 0] = 1.0
    c["w2"][0, 0, 0] = S
    c["w2"][0, 1, 0] = 1.0
    return c, lambda g: g["da"][:, 0]


def pin_da_dy_rowwise(S):
    """dA = dY . W2 (K = H): row 5 of dY holds s (h=0) and 1 (h=1) in one
    block along H; column 0 of dY holds s alone along the rows."""
    c = _base()
    c["dy"][5, 0] = S
    c["dy"][5, 1] = 1.0
    c["w2"][0, 0, 0] = 1.0
    return c, lambda g: g["da"][5:6, 0]


def pin_dx_dh1_rowwise(S):
    """dX = dH1 . W1 (K = 2F): row 3 of dH1 holds s (n=0) and 1 (n=1) along
    2F (u[3,0] = 2s, u[3,1] = 2 with dA = 1); column 0 of dH1 holds s alone."""
    c = _base()
    _unit_da(c)
    c["h1"][3, F + 0] = 2 * S
    c["h1"][3, F + 1] = 2.0
    c["w1"][0, 0, 0] = 1.0
    return c, lambda g: g["dx"][3:4, 0]


def pin_dx_w1_columnwise(S):
    """dX = dH1 . W1 (K = 2F): W1 column 0 holds s (n=0) and 1 (n=1) along
    2F; row n=0 of W1 holds s alone along H. dH1[:, 0] = 1, the rest 0."""
    c = _base()
    _unit_da(c)
    c["h1"][:, F + 0] = 2.0
    c["w1"][0, 0, 0] = S
    c["w1"][0, 1, 0] = 1.0
    return c, lambda g: g["dx"][:, 0]


def pin_dw2_dy_columnwise(S):
    """dW2 = dY^T . A (K = rows): dY column 0 holds s (row 0) and 1 (row 1)
    along the rows; row 0 of dY holds s alone along H. A[0, 0] = 1."""
    c = _base()
    c["dy"][0, 0] = S
    c["dy"][1, 0] = 1.0
    c["a"][0, 0] = 1.0
    return c, lambda g: g["dw2"][0, 0, 0:1]


def pin_dw2_a_columnwise(S):
    """dW2 = dY^T . A (K = rows): A column 0 holds s (row 0) and 1 (row 1)
    along the rows; row 0 of A holds s alone along F. dY[0, 0] = 1."""
    c = _base()
    c["a"][0, 0] = S
    c["a"][1, 0] = 1.0
    c["dy"][0, 0] = 1.0
    return c, lambda g: g["dw2"][0, 0, 0:1]


def pin_dw1_dh1_columnwise(S):
    """dW1 = dH1^T . X (K = rows): dH1 column 0 holds s (row 0) and 1 (row 1)
    along the rows (u[0,0] = 2s, u[1,0] = 2, dA = 1); row 0 of dH1 holds s
    alone along 2F. X[0, 0] = 1."""
    c = _base()
    _unit_da(c)
    c["h1"][0, F + 0] = 2 * S
    c["h1"][1, F + 0] = 2.0
    c["x"][0, 0] = 1.0
    return c, lambda g: g["dw1"][0, 0, 0:1]


def pin_dw1_x_columnwise(S):
    """dW1 = dH1^T . X (K = rows): X column 0 holds s (row 0) and 1 (row 1)
    along the rows; row 0 of X holds s alone along H. dH1[0, 0] = 1."""
    c = _base()
    _unit_da(c)
    c["h1"][0, F + 0] = 2.0
    c["x"][0, 0] = S
    c["x"][1, 0] = 1.0
    return c, lambda g: g["dw1"][0, 0, 0:1]


PINS = [pin_da_dy_rowwise, pin_da_w2_columnwise, pin_dx_dh1_rowwise, pin_dx_w1_columnwise,
        pin_dw2_dy_columnwise, pin_dw2_a_columnwise, pin_dw1_dh1_columnwise, pin_dw1_x_columnwise]


QDQ = {
    "mxfp8": lambda v: orc.dequantize_rowwise(*orc.quantize_rowwise(v)),
    "mxfp4": lambda v: orc.dequantize_rowwise_fp4(*orc.quantize_rowwise_fp4(v)),
}


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_hand_worked_block_values(fmt):
    """The two quantized values the pins rely on, from the encoder itself."""
    _, S, Q = FORMATS[fmt]
    assert QDQ[fmt](np.array([[S, 1.0] + [0.0] * 30]))[0, 0] == Q
    assert QDQ[fmt](np.array([[S] + [0.0] * 31]))[0, 0] == S
    assert QDQ[fmt](np.array([[S, 1.0, 2.0, 2 * S] + [0.0] * 28]))[0, 1:3].tolist() == [1.0, 2.0]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_operand_axis(pin, fmt):
    quantize, S, Q = FORMATS[fmt]
    c, pick = pin(S)
    got = pick(_run(c, quantize))
    assert np.all(got == Q), (pin.__name__, got)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_grouped_columnwise_blocks_restart_per_expert(fmt):
    """Experts of 31 and 9 rows: rows 30 (expert 0's last) and 31 (expert 1's
    first) would share a 32-row block of column 0 if blocks ran over all rows.
    dY[30, 0] = 1, dY[31, 0] = s, A[31, 0] = 1: expert 1's dW2[0, 0] = dY[31,0]
    quantized in expert 1's own (zero-padded) block, where s is alone: s.
    Likewise X[30, 0] = 1, X[31, 0] = s with dH1[31, 0] = 1 gives expert 1's
    dW1[0, 0] = s."""
    quantize, S, _ = FORMATS[fmt]
    c = _base(split=(31, 9))
    c["dy"][30, 0] = 1.0
    c["dy"][31, 0] = S
    c["a"][31, 0] = 1.0
    g = _run(c, quantize)
    assert g["dw2"][1, 0, 0] == S
    assert g["dw2"][0, 0, 0] == 0.0
    c = _base(split=(31, 9))
    _unit_da(c)
    c["h1"][31, F + 0] = 2.0       # dH1[31, 0] = 1 (dA = 1, g = 0)
    c["x"][30, 0] = 1.0
    c["x"][31, 0] = S
    g = _run(c, quantize)
    assert g["dw1"][1, 0, 0] == S


# -- planted mistakes: every axis swap of the backward is caught ---------------

# Call sites of the quantize-dequantize helpers in one expert's iteration of
# mlp_backward, in evaluation order: rowwise dY, columnwise W2 (dA); rowwise
# dH1, columnwise W1 (dX); columnwise dY, columnwise A (dW2); columnwise dH1,
# columnwise X (dW1).
CALL_SITES = 8


def _swap_site(monkeypatch, site):
    """Patch the oracle so that call `site` of each expert iteration quantizes
    along the other axis (a planted mistake, CPU only)."""
    row, col = mxo._qdq_row, mxo._qdq_col
    count = {"n": 0}

    def pick(native, other):
        def f(x, quantize):
            i = count["n"] % CALL_SITES
            count["n"] += 1
            return (other if i == site else native)(x, quantize)
        return f

    monkeypatch.setattr(mxo, "_qdq_row", pick(row, col))
    monkeypatch.setattr(mxo, "_qdq_col", pick(col, row))


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("site", range(CALL_SITES))
def test_each_swapped_axis_fails_a_pin(monkeypatch, site, fmt):
    quantize, S, Q = FORMATS[fmt]
    _swap_site(monkeypatch, site)
    caught = []
    for pin in PINS:
        c, pick = pin(S)
        if not np.all(pick(_run(c, quantize)) == Q):
            caught.append(pin.__name__)
    assert caught, f"swapping the axis of call site {site} passes every pin"

"""Plain float64 CPU oracle of the MXFP8 block-scaled grouped MLP.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product.

Every step follows a definition, written out directly:

* MXFP8 block quantization -- one E8M0 power-of-two scale per block of 32
  consecutive values, 8-bit E4M3 elements ("Efficient MoE training for
  biological foundation models", Key technical approaches item 2; the Llama 3
  recipe page, "MXFP8 vs BF16 throughput": MXFP8BlockScaling, E4M3).
* GroupedLinear over per-expert split_sizes (same article, item 1): each
  expert's rows are multiplied by that expert's weight; the grouped result is
  the loop of per-expert products.
* GroupedLinear -> ScaledSwiGLU -> GroupedLinear with routing-weight scaling,
  16-bit master weights quantized each step, and the corresponding backward
  (same article, item 3).

Readings where the pages are silent (each also listed in the design notes):

R1  scale exponent e = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest
    normal), floor taken exactly from the binary exponent; e clamped to
    [-127, 127]; E8M0 code = e + 127.
R2  all-zero block -> e = -127 (scale code 0x00), codes 0x00 (0x80 for -0.0).
R3  element code = E4M3 round-to-nearest, ties to the even code, of v / 2^e;
    magnitudes >= 448 saturate to 448 (0x7E), never NaN; E4M3 subnormals kept;
    the sign bit always follows the input's sign (so -tiny -> 0x80).
R4  non-finite inputs are outside the contract: the oracle raises.
R5  rowwise layout: codes [rows, cols] row-major, scales [rows, cols/32];
    blocks start at column 0; cols must be a multiple of 32.
R6  columnwise layout = rowwise layout of the transpose; with groups, each
    group's rows are zero-padded to P = ceil(m/32)*32 and group g occupies
    columns [sum_{j<g} P_j, + P_g) of a [cols, sum P] matrix; padding codes
    are 0x00 and do not change amax.
R7  weights are [out, in]: W1 [E, 2F, H] with gate rows 0..F-1 and up rows
    F..2F-1, W2 [E, H, F]; no biases.
R8  A = w_r * silu(g) * u is formed before it is requantized for GEMM2
    (routing weight applied before requantization).
R9  backward is straight-through: every GEMM runs on MXFP8 copies -- dA from
    rowwise dY and columnwise W2, dX from rowwise dH1 and columnwise W1, dW2
    from columnwise dY and A, dW1 from columnwise dH1 and X; gradients are
    E4M3 as well.  The SwiGLU backward reads H1 rounded to bf16.
R10 precisions: products and sums in float64; Y, dX and the saved H1 are
    rounded to bf16 (nearest-even from float64); dW, dprobs in float64.
R11 a zero-row expert contributes nothing; its dW is the input dW
    (accumulate) or zero (overwrite).
R12 token dispatch: the routed rows are the (token, slot) entries of the
    top-k choices, ordered by expert, then token (the per-expert groups that
    GroupedLinear takes, item 1); counts per expert are the split_sizes; an
    entry whose expert lies outside [0, E) is dropped (its perm is -1).
R14 MXFP4 (the other block-scaled MX format the pages name, run on MI355X):
    E2M1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN) with one
    E8M0 scale per 32 consecutive values; e = floor(log2 amax) - 2 (2 =
    exponent of E2M1's largest value), clamped to [-127, 127]; element =
    nearest E2M1 value of v / 2^e, ties to the even code, saturating at 6,
    sign kept (-0 -> 0x8); two codes per byte, element 2i in the low nibble.
R13 token combine: y[t] = sum over slots j of the routed output row of
    (t, j), slots with perm -1 skipped, summed in float64 and rounded once to
    bf16. The routing weight is already applied inside the MLP (R8), so the
    combine is unweighted.
R15 MXFP4 GEMM: C = A . B^T with A [m, k] and B [n, k] both rowwise MXFP4
    (R14), each element taken at its value E2M1(code) * 2^(scale - 127); the
    pages name the format's GEMMs (mxfp4 runs) but not their arithmetic, so
    the plain product of the dequantized operands is the definition.
R16 MXFP4 weight gradient: the columnwise MXFP4 layout pads each group
    (expert) to a multiple of 32 rows exactly as R6 does for MXFP8, and the
    group-K product C_g = A[:, K_g] . B[:, K_g]^T is R15 over group g's
    padded range; fp32 accumulation into an existing main gradient adds C_g.
    This is the wgrad the ROCm page says its FP4 GEMM library lacks (BF16
    output only); its arithmetic is the MXFP8 group-K form with R15's
    element values.
R17 MXFP4 MLP: the MLP of R7-R11 with every MXFP8 copy replaced by the MXFP4
    copy (R14) along the same axis -- rowwise along each forward GEMM's
    contraction axis, the straight-through backward's copies as R9 names
    them, columnwise copies padded per expert as R16 -- and every other step
    unchanged (A formed before requantization, H1 saved in bf16, Y and dX
    rounded to bf16, dW and dprobs unrounded). The Llama 3 recipe page
    assigns whole layers to FP8 or to FP4 and the ROCm page runs every layer
    of its mxfp4 model in FP4, so an FP4 layer's MLP runs its GEMMs on MXFP4
    copies; that the recipe is otherwise the MXFP8 one is the plainest
    reading. Selected by quantize="mxfp4" in the MLP functions below.
R18 NVFP4 (the 4-bit recipe the Llama 3 recipe page lists beside MXFP8, and
    whose first and last layers the ROCm page keeps in BF16; neither page
    defines its arithmetic, so this is the published form of the format):
    E2M1 elements (R14's values) in blocks of 16 consecutive values, one
    E4M3 scale per block (a positive R3 code) and one float32 scale per
    tensor. In float32 arithmetic, each step rounded to nearest even:
      S   = 2688 / amax of the whole tensor (2688 = 448 * 6, the largest
            E4M3 times the largest E2M1); amax = 0 gives S = 1, and S is
            capped at 2^64 (so that S over any block scale stays finite);
      s_b = E4M3 code (R3) of (bmax / 6) * S, bmax the block's largest
            magnitude;
      q   = E2M1 code (R14: nearest, ties to even, saturating at 6, sign kept)
            of x * (S / E4M3(s_b)); a block whose scale code is 0 gets codes
            0 (0x8 for a negative input).
    The value of element q with block scale s_b is E2M1(q) * E4M3(s_b) / S.
    The decisions (codes) are taken in float32 on both sides because they
    depend on rounding; products and sums of the GEMM are float64 here.
    Layouts: codes packed as R14 (element 2i in the low nibble), scales
    [rows, cols / 16] row-major; the columnwise copy is the rowwise copy of
    the transpose with the same S.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E8M0_BIAS = 127

__all__ = [
    "BLOCK", "E4M3_MAX", "bf16_bits_to_f64", "e4m3_value", "e8m0_value",
    "scale_exponent", "e4m3_encode", "quantize_blocks", "quantize_rowwise",
    "dequantize_rowwise", "padded_sizes", "quantize_colwise", "gemm_group_m",
    "gemm_group_k", "round_to_bf16", "sigmoid", "silu", "mlp_forward",
    "moe_dispatch", "moe_combine", "e2m1_value", "e2m1_encode", "quantize_rowwise_fp4",
    "dequantize_rowwise_fp4", "gemm_fp4", "gemm_fp4_grouped", "E2M1_VALUES",
    "mlp_backward", "mlp_forward_rows", "mlp_backward_rows",
    "mlp_backward_wgrad_entries", "quantize_colwise_fp4", "gemm_fp4_group_k",
    "NV_BLOCK", "nvfp4_tensor_scale", "quantize_rowwise_nvfp4", "quantize_colwise_nvfp4",
    "dequantize_rowwise_nvfp4", "gemm_nvfp4", "gemm_nvfp4_grouped",
]


# ---------------------------------------------------------------------------
# number formats

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_value(codes) -> np.ndarray:
    """E4M3 code -> value.  1 sign, 4 exponent (bias 7), 3 mantissa bits; no
    infinities; S.1111.111 is NaN; exponent field 0 is subnormal (m/8 * 2^-6)."""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    ef = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(ef == 0, (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2((ef - 7).astype(np.float64)))
    mag = np.where((ef == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e8m0_value(s) -> np.ndarray:
    """E8M0 code -> 2^(code - 127); code 0xFF is NaN."""
    s = np.asarray(s).astype(np.int64)
    v = np.exp2((s - E8M0_BIAS).astype(np.float64))
    return np.where(s == 255, np.nan, v)


def scale_exponent(amax) -> np.ndarray:
    """Readings R1/R2: e = floor(log2 amax) - 8 clamped to [-127, 127]; amax = 0 -> -127.

    floor(log2 a) is read off the binary exponent: a = f * 2^x with f in
    [0.5, 1) gives floor(log2 a) = x - 1 (exact, also for subnormal a)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, x = np.frexp(amax)
    e = (x.astype(np.int64) - 1) - 8
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127)


def e4m3_encode(t) -> np.ndarray:
    """Reading R3: E4M3 code of t by saturating round-to-nearest-even.

    t is float64 and already divided by the block scale.  For |t| in the
    normal range, |t| = (1 + m/8) * 2^E is solved for the integer m by rounding
    (|t| / 2^E - 1) * 8 half-to-even (all steps exact in float64); a carry to
    m = 8 moves to the next binade.  Below 2^-6 the grid is uniform with step
    2^-9, so the code is round-half-even(|t| * 2^9) (code 8 = 2^-6 is the
    smallest normal, so the two ranges join).  |t| >= 448 saturates."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    sub = a < 2.0 ** -6
    code_sub = np.rint(a * 2.0 ** 9)
    safe = np.where(sub, 1.0, a)
    _, x = np.frexp(safe)
    E = x.astype(np.int64) - 1
    frac = safe / np.exp2(E.astype(np.float64)) - 1.0
    m = np.rint(frac * 8.0).astype(np.int64)
    carry = m == 8
    E = np.where(carry, E + 1, E)
    m = np.where(carry, 0, m)
    code_norm = (E + 7) * 8 + m
    code = np.where(sub, code_sub.astype(np.int64), code_norm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.signbit(t), code | 0x80, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# block quantization

def quantize_blocks(v):
    """Quantize blocks of 32 values along the last axis -> (codes, scale codes).

    Steps: amax over the block; e per R1/R2; t = v / 2^e (exact); code per R3."""
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] != BLOCK:
        raise ValueError("last axis must be one 32-value block")
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    amax = np.max(np.abs(v), axis=-1)
    e = scale_exponent(amax)
    t = np.ldexp(v, (-e)[..., None])
    codes = e4m3_encode(t)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def quantize_rowwise(x):
    """Reading R5: rowwise MXFP8 of a [rows, cols] matrix -> (codes, scales)."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    codes, scales = quantize_blocks(x.reshape(rows, cols // BLOCK, BLOCK))
    return codes.reshape(rows, cols), scales.reshape(rows, cols // BLOCK)


def dequantize_rowwise(q, s):
    """value = E4M3(code) * 2^(scale code - 127), per 32-block along a row."""
    q = np.asarray(q)
    rows, cols = q.shape
    vals = e4m3_value(q).reshape(rows, cols // BLOCK, BLOCK)
    return (vals * e8m0_value(s)[..., None]).reshape(rows, cols)


def padded_sizes(sizes) -> np.ndarray:
    s = np.asarray(sizes, dtype=np.int64)
    return ((s + BLOCK - 1) // BLOCK) * BLOCK


def quantize_colwise(x, group_sizes=None):
    """Reading R6: columnwise MXFP8 (blocks of 32 consecutive rows per column).

    Each group's rows are zero-padded to a multiple of 32, transposed, and
    quantized rowwise; group g lands at columns [sum of earlier padded sizes,
    + its padded size) of the [cols, sum P] result."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if group_sizes is None:
        group_sizes = [rows]
    sizes = np.asarray(group_sizes, dtype=np.int64)
    if sizes.sum() != rows:
        raise ValueError("group sizes must sum to rows")
    P = padded_sizes(sizes)
    q = np.zeros((cols, int(P.sum())), dtype=np.uint8)
    s = np.zeros((cols, int(P.sum()) // BLOCK), dtype=np.uint8)
    r0 = 0
    c0 = 0
    for m, p in zip(sizes.tolist(), P.tolist()):
        if p:
            padded = np.zeros((p, cols))
            padded[:m] = x[r0:r0 + m]
            qg, sg = quantize_rowwise(padded.T)
            q[:, c0:c0 + p] = qg
            s[:, c0 // BLOCK:(c0 + p) // BLOCK] = sg
        r0 += m
        c0 += p
    return q, s


# ---------------------------------------------------------------------------
# grouped GEMM (GroupedLinear over split_sizes)

def gemm_group_m(a_q, a_s, b_q, b_s, sizes):
    """C = A_g . B_g^T for each group's rows of A (float64, dequantized operands).

    a_q [M, K] rowwise MXFP8 (M = sum of sizes); b_q [G, N, K] one weight per
    group; returns float64 [M, N]."""
    A = dequantize_rowwise(a_q, a_s)
    sizes = np.asarray(sizes, dtype=np.int64)
    G, N, K = b_q.shape
    C = np.zeros((A.shape[0], N))
    r0 = 0
    for g in range(G):
        m = int(sizes[g])
        if m:
            B = dequantize_rowwise(b_q[g], b_s[g])
            C[r0:r0 + m] = A[r0:r0 + m] @ B.T
        r0 += m
    return C


def gemm_group_k(a_q, a_s, b_q, b_s, sizes):
    """C_g = A[:, K_g] . B[:, K_g]^T, K_g = group g's padded column range.

    a_q [M, sum P], b_q [N, sum P] (columnwise-grouped MXFP8); returns
    float64 [G, M, N]; a group with no rows gives zeros."""
    A = dequantize_rowwise(a_q, a_s)
    B = dequantize_rowwise(b_q, b_s)
    P = padded_sizes(sizes)
    C = np.zeros((len(P), A.shape[0], B.shape[0]))
    k0 = 0
    for g, p in enumerate(P.tolist()):
        if p:
            C[g] = A[:, k0:k0 + p] @ B[:, k0:k0 + p].T
        k0 += p
    return C


# ---------------------------------------------------------------------------
# fused MLP

def round_to_bf16(x):
    """Round float64 to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits; with E = floor(log2|x|) (at least -126, the
    subnormal floor) the grid step is 2^(E-7)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a == 0, 1.0, a))
    E = np.maximum(ex.astype(np.int64) - 1, -126)
    q = np.exp2((E - 7).astype(np.float64))
    r = np.rint(a / q) * q
    r = np.where(r > 3.3895313892515355e38, np.inf, r)
    return np.copysign(r, x)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def _fmt(quantize):
    """The block format an MLP function's `quantize` argument names: False
    (none, float64), True or "mxfp8" (R1-R6), "mxfp4" (R14, R16, R17)."""
    if quantize is False or quantize is None:
        return None
    if quantize is True or quantize == "mxfp8":
        return "mxfp8"
    if quantize == "mxfp4":
        return "mxfp4"
    raise ValueError(f"unknown block format {quantize!r}")


def _qdq_row(x, quantize):
    f = _fmt(quantize)
    if f is None:
        return np.asarray(x, dtype=np.float64)
    if f == "mxfp4":
        return dequantize_rowwise_fp4(*quantize_rowwise_fp4(x))
    return dequantize_rowwise(*quantize_rowwise(x))


def _qdq_col(x, quantize):
    """Columnwise quantize-dequantize of one group's [m, cols] matrix, returned
    in the original [m, cols] orientation."""
    x = np.asarray(x, dtype=np.float64)
    f = _fmt(quantize)
    if f is None:
        return x
    m = x.shape[0]
    if f == "mxfp4":
        q, s = quantize_colwise_fp4(x)
        return dequantize_rowwise_fp4(q, s)[:, :m].T
    q, s = quantize_colwise(x)
    return dequantize_rowwise(q, s)[:, :m].T


def _as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def _offsets(split_sizes):
    s = np.asarray(split_sizes, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(s)])


def mlp_forward(x, probs, w1, w2, split_sizes, *, quantize=True):
    """GroupedLinear -> ScaledSwiGLU -> GroupedLinear (article item 3).

    Per expert e with rows X_e and routing weights w:
      H1 = Xq_e . W1q_e^T; g = H1[:, :F], u = H1[:, F:];
      A  = w * silu(g) * u   (R8);   Y = Aq . W2q_e^T  (rounded to bf16).
    x [R,H], w1 [E,2F,H], w2 [E,H,F] as bf16 bits or float; probs [R].
    quantize=True (or "mxfp8") runs the GEMMs on MXFP8 copies, "mxfp4" on
    MXFP4 copies (R17); False gives the unquantized float64 MLP (for
    derivative checks).
    Returns dict(y, y_exact, h1, h1_bf16, a)."""
    X = _as_f64(x)
    p = np.asarray(probs, dtype=np.float64)
    E = w1.shape[0]
    F = w1.shape[1] // 2
    off = _offsets(split_sizes)
    Xh = _qdq_row(X, quantize)
    R, H = X.shape
    H1 = np.zeros((R, 2 * F))
    A = np.zeros((R, F))
    Y = np.zeros((R, H))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        W1h = _qdq_row(_as_f64(w1[e]), quantize)
        W2h = _qdq_row(_as_f64(w2[e]), quantize)
        h1 = Xh[r0:r1] @ W1h.T
        g, u = h1[:, :F], h1[:, F:]
        a = p[r0:r1, None] * silu(g) * u
        Y[r0:r1] = _qdq_row(a, quantize) @ W2h.T
        H1[r0:r1] = h1
        A[r0:r1] = a
    return dict(y=round_to_bf16(Y), y_exact=Y, h1=H1, h1_bf16=round_to_bf16(H1), a=A)


def _swiglu_backward(dA, g, u, w):
    """Derivatives of A = w * silu(g) * u:
    dg = dA*w*u*s*(1 + g*(1-s)),  du = dA*w*silu(g),  dw = sum_f dA*silu(g)*u,
    with s = sigmoid(g) (silu'(g) = s + g*s*(1-s))."""
    s = sigmoid(g)
    sl = g * s
    dg = dA * w[:, None] * u * s * (1.0 + g * (1.0 - s))
    du = dA * w[:, None] * sl
    dw = np.sum(dA * sl * u, axis=1)
    return dg, du, dw


def mlp_backward(x, probs, w1, w2, split_sizes, dy, fwd, *, quantize=True,
                 dw1_in=None, dw2_in=None):
    """Backward of mlp_forward (article item 3, "corresponding fused backward op"),
    straight-through per reading R9.

    fwd is mlp_forward's result (its h1_bf16 and a are used; with quantize=False
    the exact h1 is used instead).  dw1_in/dw2_in, when given, are accumulated
    into (fp32 main-grad style); otherwise dW starts from zero.
    Returns dict(dx, dx_exact, dprobs, dw1, dw2, dh1, da)."""
    X = _as_f64(x)
    dY = _as_f64(dy)
    p = np.asarray(probs, dtype=np.float64)
    E = w1.shape[0]
    F = w1.shape[1] // 2
    R, H = X.shape
    off = _offsets(split_sizes)
    h1 = fwd["h1_bf16"] if _fmt(quantize) else fwd["h1"]
    A = fwd["a"]
    dX = np.zeros((R, H))
    dP = np.zeros(R)
    dH1 = np.zeros((R, 2 * F))
    dAll = np.zeros((R, F))
    dW1 = np.zeros(w1.shape) if dw1_in is None else np.array(dw1_in, dtype=np.float64)
    dW2 = np.zeros(w2.shape) if dw2_in is None else np.array(dw2_in, dtype=np.float64)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        W1 = _as_f64(w1[e])
        W2 = _as_f64(w2[e])
        dA = _qdq_row(dY[r0:r1], quantize) @ _qdq_col(W2, quantize)
        g, u = h1[r0:r1, :F], h1[r0:r1, F:]
        dg, du, dw = _swiglu_backward(dA, g, u, p[r0:r1])
        dh = np.concatenate([dg, du], axis=1)
        dX[r0:r1] = _qdq_row(dh, quantize) @ _qdq_col(W1, quantize)
        dW2[e] += _qdq_col(dY[r0:r1], quantize).T @ _qdq_col(A[r0:r1], quantize)
        dW1[e] += _qdq_col(dh, quantize).T @ _qdq_col(X[r0:r1], quantize)
        dP[r0:r1] = dw
        dH1[r0:r1] = dh
        dAll[r0:r1] = dA
    return dict(dx=round_to_bf16(dX), dx_exact=dX, dprobs=dP, dw1=dW1, dw2=dW2, dh1=dH1,
                da=dAll)


# ---------------------------------------------------------------------------
# sampled evaluation at full size (same steps, restricted to chosen outputs)

def _expert_of_rows(split_sizes, rows):
    off = _offsets(split_sizes)
    return np.searchsorted(off, np.asarray(rows), side="right") - 1


def mlp_forward_rows(x, probs, w1, w2, split_sizes, rows, quantize=True):
    """Y (bf16-rounded) and A for the selected rows only (quantize names the
    block format as in mlp_forward).

    Rowwise quantization acts on one row at a time, so a row's Y depends only
    on that row, its routing weight and its expert's weights."""
    rows = np.asarray(rows, dtype=np.int64)
    F = w1.shape[1] // 2
    H = w1.shape[2]
    ex = _expert_of_rows(split_sizes, rows)
    Y = np.zeros((len(rows), H))
    A = np.zeros((len(rows), F))
    H1 = np.zeros((len(rows), 2 * F))
    p = np.asarray(probs, dtype=np.float64)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        r = rows[sel]
        Xh = _qdq_row(_as_f64(x[r]), quantize)
        W1h = _qdq_row(_as_f64(w1[e]), quantize)
        h1 = Xh @ W1h.T
        del W1h
        a = p[r, None] * silu(h1[:, :F]) * h1[:, F:]
        W2h = _qdq_row(_as_f64(w2[e]), quantize)
        Y[sel] = _qdq_row(a, quantize) @ W2h.T
        A[sel] = a
        H1[sel] = h1
    return dict(y=round_to_bf16(Y), a=A, h1_bf16=round_to_bf16(H1))


def _expert_dh1(x, probs, w1, w2, split_sizes, dy, e, r_sel=None, quantize=True):
    """dH1 rows of expert e (all its rows, or the positions r_sel within it),
    from the fwd's bf16 H1 and the straight-through dA.  Also returns dprobs of
    those rows and the unrounded H1 (from which the forward formed A)."""
    off = _offsets(split_sizes)
    r0, r1 = int(off[e]), int(off[e + 1])
    F = w1.shape[1] // 2
    idx = np.arange(r0, r1) if r_sel is None else r0 + np.asarray(r_sel)
    Xh = _qdq_row(_as_f64(x[idx]), quantize)
    W1h = _qdq_row(_as_f64(w1[e]), quantize)
    h1 = Xh @ W1h.T
    del W1h
    hb = round_to_bf16(h1)
    dA = _qdq_row(_as_f64(dy[idx]), quantize) @ _qdq_col(_as_f64(w2[e]), quantize)
    p = np.asarray(probs, dtype=np.float64)[idx]
    dg, du, dw = _swiglu_backward(dA, hb[:, :F], hb[:, F:], p)
    return np.concatenate([dg, du], axis=1), dw, h1


def mlp_backward_rows(x, probs, w1, w2, split_sizes, dy, rows, quantize=True):
    """dX (bf16-rounded) and dprobs for the selected rows only."""
    rows = np.asarray(rows, dtype=np.int64)
    off = _offsets(split_sizes)
    ex = _expert_of_rows(split_sizes, rows)
    H = w1.shape[2]
    dX = np.zeros((len(rows), H))
    dP = np.zeros(len(rows))
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        dh, dw, _ = _expert_dh1(x, probs, w1, w2, split_sizes, dy, e,
                                rows[sel] - int(off[e]), quantize)
        dX[sel] = _qdq_row(dh, quantize) @ _qdq_col(_as_f64(w1[e]), quantize)
        dP[sel] = dw
    return dict(dx=round_to_bf16(dX), dprobs=dP)


def mlp_backward_wgrad_entries(x, probs, w1, w2, split_sizes, dy, expert,
                               dw1_idx, dw2_idx, quantize=True):
    """Selected entries of one expert's dW1 (indices (n, h)) and dW2 ((h, f)),
    from a zero start.

    Every quantization on the way is per row over the contraction axis (X, dY,
    W1 rows) or per column over the expert's rows (W2 over H, dH1, A, X and dY
    for the weight gradients), so an entry only needs the columns it touches:
    ffn column c = n mod F of H1 (gate c and up F + c) and dA for dW1, gate
    and up column f of H1 for dW2, and columns h of X and dY. The arithmetic
    per column is that of _expert_dh1 / mlp_backward."""
    off = _offsets(split_sizes)
    r0, r1 = int(off[expert]), int(off[expert + 1])
    F = w1.shape[1] // 2
    dw1_idx = np.asarray(dw1_idx, dtype=np.int64).reshape(-1, 2)
    dw2_idx = np.asarray(dw2_idx, dtype=np.int64).reshape(-1, 2)
    if r1 == r0:
        return np.zeros(len(dw1_idx)), np.zeros(len(dw2_idx))
    p = np.asarray(probs, dtype=np.float64)[r0:r1]
    Xh = _qdq_row(_as_f64(x[r0:r1]), quantize)
    dYh = _qdq_row(_as_f64(dy[r0:r1]), quantize)

    def h1_cols(cs):
        """Unrounded gate and up columns cs of H1 = Xh . W1h^T."""
        W1h_g = _qdq_row(_as_f64(w1[expert][cs]), quantize)
        W1h_u = _qdq_row(_as_f64(w1[expert][F + cs]), quantize)
        return Xh @ W1h_g.T, Xh @ W1h_u.T

    # dW1[n, h] = sum_r dH1c[r, n] * Xc[r, h]
    c1 = np.unique(dw1_idx[:, 0] % F)
    g, u = h1_cols(c1)
    dA = dYh @ _qdq_col(_as_f64(w2[expert][:, c1]), quantize)
    dg, du, _ = _swiglu_backward(dA, round_to_bf16(g), round_to_bf16(u), p)
    dh = np.concatenate([dg, du], axis=1)                     # columns c1, then F + c1
    dh_pos = {int(c): i for i, c in enumerate(c1.tolist())}
    dh_pos.update({int(F + c): len(c1) + i for i, c in enumerate(c1.tolist())})
    n_sel = np.unique(dw1_idx[:, 0])
    dhc = _qdq_col(dh[:, [dh_pos[int(n)] for n in n_sel]], quantize)
    h_sel = np.unique(dw1_idx[:, 1])
    xc = _qdq_col(_as_f64(x[r0:r1][:, h_sel]), quantize)
    n_map = {int(n): i for i, n in enumerate(n_sel.tolist())}
    h_map = {int(h): i for i, h in enumerate(h_sel.tolist())}
    out1 = np.array([dhc[:, n_map[n]] @ xc[:, h_map[h]] for n, h in dw1_idx.tolist()])

    # dW2[h, f] = sum_r dYc[r, h] * Ac[r, f], A = w * silu(gate) * up (unrounded H1)
    f_sel = np.unique(dw2_idx[:, 1])
    g2, u2 = h1_cols(f_sel)
    ac = _qdq_col(p[:, None] * silu(g2) * u2, quantize)
    h2_sel = np.unique(dw2_idx[:, 0])
    dyc = _qdq_col(_as_f64(dy[r0:r1][:, h2_sel]), quantize)
    h2_map = {int(h): i for i, h in enumerate(h2_sel.tolist())}
    f_map = {int(f): i for i, f in enumerate(f_sel.tolist())}
    out2 = np.array([dyc[:, h2_map[h]] @ ac[:, f_map[f]] for h, f in dw2_idx.tolist()])
    return out1, out2


# ---------------------------------------------------------------------------
# token dispatch and combine around the grouped MLP (R12, R13)
# ("Efficient MoE training for biological foundation models": "Dense vs. MoE
# scaling" -- each token activates a few experts and routing adds overhead;
# "Key technical approaches" item 1 -- GroupedLinear gathers the input tokens
# of each expert and takes per-expert token counts, split_sizes)

def moe_dispatch(x, topk_idx, topk_w, num_experts):
    """Gather each token's rows into per-expert groups (R12).

    x: [T, H] (any dtype, copied as is); topk_idx int [T, k]; topk_w [T, k]
    or None. Returns dict: x_perm [R, H] (R = valid entries), probs_perm
    float32 [R] (or None), perm int32 [T, k] (routed row of entry (t, j), -1
    if dropped), row_token int32 [R], counts int64 [E]."""
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    entries = []                       # (t, j) in routed-row order
    for e in range(num_experts):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    entries.append((t, j))
    R = len(entries)
    perm = np.full((T, k), -1, dtype=np.int32)
    row_token = np.empty(R, dtype=np.int32)
    for r, (t, j) in enumerate(entries):
        perm[t, j] = r
        row_token[r] = t
    counts = np.zeros(num_experts, dtype=np.int64)
    for (t, j) in entries:
        counts[idx[t, j]] += 1
    x = np.asarray(x)
    x_perm = x[row_token] if R else np.empty((0,) + x.shape[1:], dtype=x.dtype)
    probs = None
    if topk_w is not None:
        w = np.asarray(topk_w, dtype=np.float32)
        probs = np.array([w[t, j] for (t, j) in entries], dtype=np.float32)
    return dict(x_perm=x_perm, probs_perm=probs, perm=perm, row_token=row_token, counts=counts)


def moe_combine(y_perm_bits, perm):
    """y[t] = bf16(sum_j y_perm[perm[t, j]]) over the valid slots (R13).
    y_perm_bits: bf16 bit patterns [R, H]. Returns the bf16 values [T, H] as
    float64."""
    perm = np.asarray(perm)
    T, k = perm.shape
    y = bf16_bits_to_f64(y_perm_bits)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if perm[t, j] >= 0:
                out[t] += y[perm[t, j]]
    return round_to_bf16(out)


# ---------------------------------------------------------------------------
# MXFP4 (R14): E2M1 elements with one E8M0 scale per 32 values

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_value(codes) -> np.ndarray:
    """E2M1 code (4 bits) -> value: exponent field 0 is subnormal (m * 0.5),
    otherwise (1 + m/2) * 2^(field - 1); bit 3 is the sign."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    ef = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(ef == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2((ef - 1).astype(np.float64)))
    return np.where((c >> 3) == 1, -mag, mag)


def e2m1_encode(t) -> np.ndarray:
    """Nearest E2M1 value of t (already divided by the block scale), ties to
    the even code, saturating at 6; the sign bit follows t (R14). Written as
    the definition: distance to each of the 8 magnitudes, smallest wins, an
    equal distance goes to the even code."""
    t = np.asarray(t, dtype=np.float64)
    flat = t.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 22                                      # elements per pass (bounds the 8-way distance table)
    for i in range(0, flat.size, step):
        c = flat[i:i + step]
        d = np.abs(np.abs(c)[:, None] - E2M1_VALUES)
        best = np.argmin(d, axis=-1)                    # first (lower) code on a tie
        dmin = np.take_along_axis(d, best[:, None], axis=-1)[:, 0]
        nxt = np.minimum(best + 1, 7)
        tie = (np.take_along_axis(d, nxt[:, None], axis=-1)[:, 0] == dmin) & (nxt != best)
        code = np.where(tie & (best % 2 == 1), nxt, best)
        out[i:i + step] = code | np.where(np.signbit(c), 8, 0)
    return out.reshape(t.shape)


def quantize_rowwise_fp4(x):
    """Rowwise MXFP4 of [rows, cols] (cols % 32 == 0) -> (packed codes
    [rows, cols/2] uint8, scales [rows, cols/32] uint8)."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    v = x.reshape(rows, cols // BLOCK, BLOCK)
    amax = np.max(np.abs(v), axis=-1)
    _, ex = np.frexp(amax)
    e = np.where(amax == 0.0, -127, (ex.astype(np.int64) - 1) - 2)
    e = np.clip(e, -127, 127)
    codes = e2m1_encode(np.ldexp(v, (-e)[..., None])).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + E8M0_BIAS).astype(np.uint8)


def dequantize_rowwise_fp4(q, s):
    """value = E2M1(code) * 2^(scale code - 127); low nibble = even element."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    scale = np.repeat(e8m0_value(s), BLOCK, axis=1)
    return e2m1_value(codes) * scale


def gemm_fp4(a_q, a_s, b_q, b_s):
    """C = A . B^T (float64) for rowwise MXFP4 operands A [m, k], B [n, k]:
    each operand dequantized by the MX rule (element times its block's
    2^(scale code - 127)), then one matmul. The GEMM of the 4-bit MX runs
    ("examples/llama: default-on fusion & DP-comm perf toggles")."""
    return dequantize_rowwise_fp4(a_q, a_s) @ dequantize_rowwise_fp4(b_q, b_s).T


def gemm_fp4_grouped(a_q, a_s, b_q, b_s, sizes):
    """GroupedLinear at MXFP4 (R15 per group): the rows of A split into
    consecutive groups of sizes[g] rows ("Efficient MoE training for
    biological foundation models", Key technical approaches item 1); group g's
    rows times B_g^T, b_q [G, n, k/2]. Returns float64 [sum(sizes), n]."""
    sizes = [int(v) for v in sizes]
    G, n = b_q.shape[0], b_q.shape[1]
    C = np.zeros((sum(sizes), n))
    r0 = 0
    for g in range(G):
        if sizes[g]:
            C[r0:r0 + sizes[g]] = gemm_fp4(a_q[r0:r0 + sizes[g]], a_s[r0:r0 + sizes[g]], b_q[g], b_s[g])
        r0 += sizes[g]
    return C


def quantize_colwise_fp4(x, group_sizes=None):
    """Columnwise MXFP4 with per-group padding, the 4-bit form of R6: each
    group's rows are zero-padded to a multiple of 32, transposed and quantized
    rowwise (R14); group g occupies columns [sum of earlier padded sizes,
    + its padded size) of the [cols, sum P] result. Returns (packed codes
    [cols, sum P / 2], scales [cols, sum P / 32])."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if group_sizes is None:
        group_sizes = [rows]
    sizes = np.asarray(group_sizes, dtype=np.int64)
    if sizes.sum() != rows:
        raise ValueError("group sizes must sum to rows")
    P = padded_sizes(sizes)
    q = np.zeros((cols, int(P.sum()) // 2), dtype=np.uint8)
    s = np.zeros((cols, int(P.sum()) // BLOCK), dtype=np.uint8)
    r0 = 0
    c0 = 0
    for m, p in zip(sizes.tolist(), P.tolist()):
        if p:
            padded = np.zeros((p, cols))
            padded[:m] = x[r0:r0 + m]
            qg, sg = quantize_rowwise_fp4(padded.T)
            q[:, c0 // 2:(c0 + p) // 2] = qg
            s[:, c0 // BLOCK:(c0 + p) // BLOCK] = sg
        r0 += m
        c0 += p
    return q, s


def gemm_fp4_group_k(a_q, a_s, b_q, b_s, sizes):
    """The weight-gradient form at MXFP4: C_g = A[:, K_g] . B[:, K_g]^T with
    K_g group g's padded column range (the columnwise layout above), for
    A [M, sum P] and B [N, sum P] packed MXFP4 operands. Returns float64
    [G, M, N]; a group with no rows gives zeros."""
    A = dequantize_rowwise_fp4(a_q, a_s)
    B = dequantize_rowwise_fp4(b_q, b_s)
    P = padded_sizes(sizes)
    C = np.zeros((len(P), A.shape[0], B.shape[0]))
    k0 = 0
    for g, p in enumerate(P.tolist()):
        if p:
            C[g] = A[:, k0:k0 + p] @ B[:, k0:k0 + p].T
        k0 += p
    return C


# ---------------------------------------------------------------------------
# NVFP4 (R18): E2M1 elements, one E4M3 scale per 16 values, one float32
# scale per tensor

NV_BLOCK = 16
NVFP4_RANGE = np.float32(448.0 * 6.0)
NVFP4_SCALE_CAP = np.float32(2.0 ** 64)


def nvfp4_tensor_scale(amax) -> np.float32:
    """R18: S = 2688 / amax in float32 (one rounding), 1 for amax = 0, at most 2^64."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore"):
        q = np.float32(NVFP4_RANGE / a)
    return np.float32(min(q, NVFP4_SCALE_CAP))


def quantize_rowwise_nvfp4(x, amax=None):
    """Rowwise NVFP4 of [rows, cols] (cols % 16 == 0; values exact in
    float32) -> (packed codes [rows, cols/2] uint8, E4M3 block-scale codes
    [rows, cols/16] uint8, amax float32). The steps of R18 in order, each a
    float32 operation. amax: the whole tensor's amax when x holds only some
    of its rows (default: x's own)."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % NV_BLOCK:
        raise ValueError("cols must be a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    xf = x.astype(np.float32)
    if not np.array_equal(xf.astype(np.float64), x):
        raise ValueError("inputs must be exact float32 values")
    if amax is None:
        amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0.0)
    amax = np.float32(amax)
    S = nvfp4_tensor_scale(amax)
    v = xf.reshape(rows, cols // NV_BLOCK, NV_BLOCK)
    bmax = np.max(np.abs(v), axis=-1)
    t = (bmax / np.float32(6.0)).astype(np.float32)
    sb = (t * S).astype(np.float32)
    sc = e4m3_encode(sb.astype(np.float64))
    sv = e4m3_value(sc).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(sv > 0, S / np.where(sv > 0, sv, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    y = (v * r[..., None]).astype(np.float32)
    codes = e2m1_encode(y.astype(np.float64)).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc.astype(np.uint8), amax


def quantize_colwise_nvfp4(x):
    """Columnwise NVFP4 (R18): the rowwise copy of the transpose, blocks of 16
    consecutive rows per column (rows % 16 == 0), same tensor scale."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] % NV_BLOCK:
        raise ValueError("rows must be a multiple of 16")
    return quantize_rowwise_nvfp4(x.T)


def dequantize_rowwise_nvfp4(q, s, amax):
    """value = E2M1(code) * E4M3(block scale) / S (float64), S from amax (R18)."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    scale = np.repeat(e4m3_value(s), NV_BLOCK, axis=1)
    return e2m1_value(codes) * scale / np.float64(nvfp4_tensor_scale(amax))


def gemm_nvfp4(a_q, a_s, a_amax, b_q, b_s, b_amax):
    """C = A . B^T (float64) for rowwise NVFP4 operands A [m, k], B [n, k],
    each element at its R18 value; the plain product of the dequantized
    operands is the definition."""
    return dequantize_rowwise_nvfp4(a_q, a_s, a_amax) @ dequantize_rowwise_nvfp4(b_q, b_s, b_amax).T


def gemm_nvfp4_grouped(a_q, a_s, a_amax, b_q, b_s, b_amax, sizes):
    """GroupedLinear at NVFP4: consecutive groups of sizes[g] rows of A times
    B_g^T, each group's weight B_g with its own tensor scale (b_amax[g]).
    Returns float64 [sum(sizes), n]."""
    sizes = [int(v) for v in sizes]
    n = b_q.shape[1]
    C = np.zeros((sum(sizes), n))
    A = dequantize_rowwise_nvfp4(a_q, a_s, a_amax)
    r0 = 0
    for g, m in enumerate(sizes):
        if m:
            C[r0:r0 + m] = A[r0:r0 + m] @ dequantize_rowwise_nvfp4(b_q[g], b_s[g], b_amax[g]).T
        r0 += m
    return C

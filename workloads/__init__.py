"""Seeded synthetic inputs for the MXFP8 grouped MLP.

This module is shared by the tests, the bench and the checks that call the
oracle.  It holds none of the method's arithmetic: only random draws, the
rounding of those draws to bf16 storage, and the routing bookkeeping that turns
random router logits into per-expert row counts (``split_sizes``) and routing
weights.  Both the HIP path and the oracle receive the same bytes from here.

Recipe (fixed draw order per workload: X, W1, W2, logits, bias, dY):

* values are drawn with ``numpy.random.default_rng(seed)`` in float32
  (Student-t in float64), then rounded to bf16 by round-to-nearest-even on the
  float32 bit pattern; arrays are returned as ``uint16`` bf16 bit patterns;
* activations ~ N(0, 1), weights ~ N(0, 0.02), output gradients ~ N(0, 1e-3);
* routing: logits ~ N(0, 1) per (token, expert) plus a per-expert bias
  ~ N(0, 1); each token picks its top-2 experts (lower index wins an exact
  tie); routed rows are ordered by (expert, token); a row's weight is the
  softmax over the token's two selected (biased) logits, stored as float32.

The five named workloads follow the shapes of the Llama-3.1-8B MLP
(hidden 4096, ffn 14336) and of a Mixtral-8x7B-shaped MoE layer (8 experts,
top-2), plus a tiny MoE case and a standalone quantize tensor.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "normal_bf16", "route_top2", "make_mlp_inputs", "quantize_tensor_c2",
    "small_mlp_case", "random_mx_operand",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    tokens: int          # tokens before top-k routing
    topk: int
    experts: int
    hidden: int
    ffn: int
    backward: bool
    description: str

    @property
    def rows(self) -> int:
        return self.tokens * self.topk


WORKLOADS = {
    "tiny_moe_fwd": Workload(
        "tiny_moe_fwd", 1, 256, 2, 4, 256, 512, False,
        "tiny MoE MLP fwd: 256 tokens top-2 of 4 experts (512 rows), H=256, "
        "F=512, one expert forced empty"),
    "quantize_16384x4096": Workload(
        "quantize_16384x4096", 2, 16384, 1, 1, 4096, 0, False,
        "standalone quantize of a 16384x4096 bf16 Student-t(3) tensor with "
        "0.1% outliers x1000 and 1% all-zero 32x32 tiles"),
    "llama8b_dense_fwd": Workload(
        "llama8b_dense_fwd", 3, 8192, 1, 1, 4096, 14336, False,
        "Llama-3.1-8B dense MLP fwd: M=8192 (mbs 2 x seq 4096), H=4096, "
        "F=14336, routing weight 1"),
    "mixtral_moe_fwd": Workload(
        "mixtral_moe_fwd", 4, 8192, 2, 8, 4096, 14336, False,
        "Mixtral-8x7B-shaped MoE MLP fwd: 8192 tokens top-2 of 8 (16384 rows), "
        "H=4096, F=14336"),
    "mixtral_moe_fwd_bwd": Workload(
        "mixtral_moe_fwd_bwd", 5, 4096, 2, 8, 4096, 14336, True,
        "Mixtral-8x7B-shaped MoE MLP fwd+bwd: 4096 tokens top-2 of 8 "
        "(8192 rows), H=4096, F=14336, dY ~ N(0, 1e-3)"),
}


# ---------------------------------------------------------------------------
# bf16 storage of draws

def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0,
                chunk_rows: int = 4096) -> np.ndarray:
    """N(0, std^2) draws stored as bf16 bits, generated in row chunks to bound memory."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        v = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[r0:r1] = bf16_bits_from_f32(v)
    return out


# ---------------------------------------------------------------------------
# routing bookkeeping (produces split_sizes and routing weights)

def top2_picks(logits: np.ndarray, bias: np.ndarray):
    """The two experts each token picks (by biased logit, lower index wins ties)
    and their routing weights (softmax over the two picks).

    Returns (idx int32 [T, 2], w float32 [T, 2])."""
    z = logits + bias[None, :]
    order = np.argsort(-z, axis=1, kind="stable")[:, :2]          # lower index wins ties
    sel = np.take_along_axis(z, order, axis=1)                    # [T, 2]
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)                        # softmax over the two picks
    return order.astype(np.int32), w.astype(np.float32)


def route_top2(logits: np.ndarray, bias: np.ndarray):
    """Top-2 routing of each token.

    Returns (split_sizes int64[E], token_of_row int64[R], probs float32[R]) with
    rows ordered by (expert, token)."""
    T, E = logits.shape
    order, w = top2_picks(logits, bias)
    expert = order.reshape(-1).astype(np.int64)
    token = np.repeat(np.arange(T), 2)
    weight = w.reshape(-1)
    key = expert * T + token
    perm = np.argsort(key, kind="stable")
    split = np.bincount(expert, minlength=E).astype(np.int64)
    return split, token[perm].astype(np.int64), weight[perm].astype(np.float32)


def _tiny_split(rng: np.random.Generator, rows: int, experts: int, empty: int):
    """Multinomial split with one expert forced empty; redraw if any expert exceeds
    half of the rows (top-2 routing cannot give an expert more rows than tokens)."""
    p = np.full(experts, 1.0 / (experts - 1))
    p[empty] = 0.0
    while True:
        s = rng.multinomial(rows, p).astype(np.int64)
        if s.max() <= rows // 2:
            return s


def make_mlp_inputs(wl: Workload, *, with_dy: bool | None = None):
    """Inputs of one grouped-MLP workload as numpy arrays (bf16 as uint16 bits).

    Keys: x [R,H], w1 [E,2F,H] (gate rows first, then up rows), w2 [E,H,F],
    split_sizes int64[E], probs float32[R], and dy [R,H] when the workload has a
    backward pass (or with_dy=True)."""
    rng = np.random.default_rng(wl.seed)
    R, E, H, F = wl.rows, wl.experts, wl.hidden, wl.ffn
    x = normal_bf16(rng, (R, H), 1.0)
    w1 = normal_bf16(rng, (E, 2 * F, H), 0.02)
    w2 = normal_bf16(rng, (E, H, F), 0.02)
    if E == 1:
        split = np.array([R], dtype=np.int64)
        probs = np.ones(R, dtype=np.float32)
    elif wl.name == "tiny_moe_fwd":
        split = _tiny_split(rng, R, E, empty=1)
        d = rng.standard_normal(R)                       # per-row logit gap of the top-2 pair
        probs = (1.0 / (1.0 + np.exp(-d))).astype(np.float32)
    else:
        logits = rng.standard_normal((wl.tokens, E))
        bias = rng.standard_normal(E)
        split, _, probs = route_top2(logits, bias)
    out = dict(x=x, w1=w1, w2=w2, split_sizes=split, probs=probs)
    if with_dy if with_dy is not None else wl.backward:
        out["dy"] = normal_bf16(rng, (R, H), 1e-3)
    return out


def make_dispatch_inputs(tokens: int, experts: int, hidden: int, seed: int):
    """Tokens and top-2 routing for token dispatch / combine: x bf16 bits
    [T, H] ~ N(0,1), logits N(0,1) plus a per-expert bias N(0,1) (skewed
    expert loads, as the Mixtral-shaped workloads). Returns dict with x,
    topk_idx int32 [T, 2], topk_w float32 [T, 2], and y_perm bf16 bits
    [2T, H] ~ N(0,1) standing in for the MLP's routed output."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (tokens, hidden), 1.0)
    logits = rng.standard_normal((tokens, experts))
    bias = rng.standard_normal(experts)
    idx, w = top2_picks(logits, bias)
    y_perm = normal_bf16(rng, (2 * tokens, hidden), 1.0)
    return dict(x=x, topk_idx=idx, topk_w=w, y_perm=y_perm, logits=logits, bias=bias)


def quantize_tensor_c2(seed: int = 2, rows: int = 16384, cols: int = 4096):
    """Student-t(3) bf16 tensor with 0.1% outliers (x1000) and 1% zeroed 32x32 tiles."""
    rng = np.random.default_rng(seed)
    v = rng.standard_t(3, size=(rows, cols))
    n_out = (rows * cols) // 1000
    idx = rng.choice(rows * cols, size=n_out, replace=False)
    v.reshape(-1)[idx] *= 1000.0
    tr, tc = rows // 32, cols // 32
    nz = max(1, (tr * tc) // 100)
    tiles = rng.choice(tr * tc, size=nz, replace=False)
    v4 = v.reshape(tr, 32, tc, 32)
    v4[tiles // tc, :, tiles % tc, :] = 0.0
    return bf16_bits_from_f32(v.astype(np.float32))


def small_mlp_case(seed: int, experts: int, hidden: int, ffn: int,
                   split_sizes, *, probs: str = "random"):
    """Small grouped-MLP inputs for parity tests (explicit split_sizes).

    probs: "random" (uniform in (0,1)), "one" (all 1) or "zero" (all 0)."""
    rng = np.random.default_rng(seed)
    split = np.asarray(split_sizes, dtype=np.int64)
    R = int(split.sum())
    x = normal_bf16(rng, (R, hidden), 1.0)
    w1 = normal_bf16(rng, (experts, 2 * ffn, hidden), 0.02)
    w2 = normal_bf16(rng, (experts, hidden, ffn), 0.02)
    if probs == "random":
        p = rng.uniform(0.05, 1.0, size=R).astype(np.float32)
    elif probs == "one":
        p = np.ones(R, dtype=np.float32)
    elif probs == "zero":
        p = np.zeros(R, dtype=np.float32)
    else:
        raise ValueError(probs)
    dy = normal_bf16(rng, (R, hidden), 1e-3)
    return dict(x=x, w1=w1, w2=w2, split_sizes=split, probs=p, dy=dy)


def random_mx_operand(rng: np.random.Generator, rows: int, cols: int,
                      scale_lo: int = 120, scale_hi: int = 134):
    """Random MXFP8 operand: E4M3 codes (NaN codes excluded) and E8M0 scales.

    Returns (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    c = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] &= 0xFE
    s = rng.integers(scale_lo, scale_hi + 1, size=(rows, cols // 32), dtype=np.uint8)
    return c, s

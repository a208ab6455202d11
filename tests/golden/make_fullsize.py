"""Expected values for the full-size grouped-MLP parity tests, from the oracle only.

For each full-size workload (inputs regenerated from the workload's seed by
workloads.make_mlp_inputs) the oracle evaluates a sample of outputs it can
compute one by one, for EVERY non-empty expert: Y at its first row, its last
row, a row inside its last partial 32-row block (the block that the grouped
columnwise layouts zero-pad) and one random row; for a workload with a
backward, dX and dprobs at the same rows and entries of every non-empty
expert's dW1 and dW2 (from a zero start; each expert's contraction runs over
its own columnwise blocks). The sample and the values go to
fullsize_<workload>.npz beside this script; with --mxfp4, the same sample
of the MLP whose GEMMs run on MXFP4 copies (the oracle's quantize="mxfp4",
reading R17) goes to fullsize_<workload>_mxfp4.npz.

    python tests/golden/make_fullsize.py [--mxfp4] [workload ...]

Each workload takes minutes of CPU (the exact float64 quantizer runs over
whole expert weight matrices for the sampled rows of every expert).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as orc  # noqa: E402
import workloads as wl  # noqa: E402

FULLSIZE = ("llama8b_dense_fwd", "mixtral_moe_fwd", "mixtral_moe_fwd_bwd")
ENTRIES_PER_EXPERT = 24


def golden_path(name: str, fmt: str = "mxfp8") -> str:
    suffix = "" if fmt == "mxfp8" else f"_{fmt}"
    return os.path.join(HERE, f"fullsize_{name}{suffix}.npz")


def make(name: str, fmt: str = "mxfp8") -> str:
    quantize = True if fmt == "mxfp8" else fmt
    w = wl.WORKLOADS[name]
    t0 = time.time()
    c = wl.make_mlp_inputs(w, with_dy=w.backward)
    split = np.asarray(c["split_sizes"], dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(split)])
    F, H = w.ffn, w.hidden
    experts = [e for e in range(w.experts) if split[e] > 0]
    rng = np.random.default_rng(1000 + w.seed)
    rows = []
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        pick = {r0, r1 - 1, int(rng.integers(r0, r1))}
        m = r1 - r0
        if m % 32:                                   # a row inside the last, partial 32-row block
            pick.add(int(rng.integers(r0 + m // 32 * 32, r1)))
        rows += sorted(pick)
    rows = np.asarray(rows, dtype=np.int64)
    out = dict(workload=np.array(name), fmt=np.array(fmt), split=split,
               experts=np.asarray(experts, dtype=np.int64), rows=rows)

    f = orc.mlp_forward_rows(c["x"], c["probs"], c["w1"], c["w2"], split, rows, quantize)
    out["y"] = f["y"]
    print(f"[{name} {fmt}] forward rows done ({time.time() - t0:.0f} s)", flush=True)
    if w.backward:
        b = orc.mlp_backward_rows(c["x"], c["probs"], c["w1"], c["w2"], split, c["dy"], rows, quantize)
        out["dx"], out["dprobs"] = b["dx"], b["dprobs"]
        print(f"[{name} {fmt}] backward rows done ({time.time() - t0:.0f} s)", flush=True)
        i1, v1, i2, v2 = [], [], [], []
        for e in experts:
            n = rng.integers(0, 2 * F, ENTRIES_PER_EXPERT)
            n[: ENTRIES_PER_EXPERT // 2] %= F            # half gate rows, the rest anywhere
            h = rng.integers(0, H, ENTRIES_PER_EXPERT)
            d1 = np.stack([n, h], axis=1)
            d2 = np.stack([rng.integers(0, H, ENTRIES_PER_EXPERT), rng.integers(0, F, ENTRIES_PER_EXPERT)], axis=1)
            a1, a2 = orc.mlp_backward_wgrad_entries(c["x"], c["probs"], c["w1"], c["w2"], split,
                                                    c["dy"], e, d1, d2, quantize)
            i1.append(np.concatenate([np.full((len(d1), 1), e), d1], axis=1)); v1.append(a1)
            i2.append(np.concatenate([np.full((len(d2), 1), e), d2], axis=1)); v2.append(a2)
        out["dw1_idx"], out["dw1"] = np.concatenate(i1), np.concatenate(v1)
        out["dw2_idx"], out["dw2"] = np.concatenate(i2), np.concatenate(v2)
        print(f"[{name} {fmt}] weight-gradient entries done ({time.time() - t0:.0f} s)", flush=True)
    path = golden_path(name, fmt)
    np.savez_compressed(path, **out)
    print(f"[{name} {fmt}] wrote {path}", flush=True)
    return path


if __name__ == "__main__":
    args = sys.argv[1:]
    fmt = "mxfp4" if "--mxfp4" in args else "mxfp8"
    names = [a for a in args if not a.startswith("--")]
    for nm in names or (FULLSIZE if fmt == "mxfp8" else ("mixtral_moe_fwd_bwd",)):
        make(nm, fmt)

"""Layer-wise precision selection (host logic only; no device work).

"TransformerEngine-accelerated Llama 3 training with native PyTorch training
loop", section Layer-Wise Precision: the layers that run in FP8 and in FP4
are named by 1-indexed layer numbers (fp8_layers, fp4_layers); layers named
by neither run in BF16; when both formats are enabled and only one list is
given, the other format takes every remaining layer.

"examples/llama: default-on fusion & DP-comm perf toggles - #141", section
Changes: the FP4 default is recipe-aware: with mxfp4 every layer runs in FP4;
with nvfp4 the first and the last layer stay in BF16.

Readings where the pages leave a case open (stated, not quoted):
  - both formats enabled and neither list given: the FP4 recipe's default
    layers run in FP4 and FP8 takes the rest (the rule "the other format
    claims the remaining layers", applied to the FP4 default);
  - one format enabled without a list: every layer for FP8; the recipe's
    default layers for FP4;
  - a list for a format that is not enabled, a layer number outside
    1..num_layers, a repeated layer, or a layer in both lists: ValueError.

The FP8 format of this library is MXFP8 block scaling; FP4 is MXFP4 (the
format the gfx950 scaled MFMA runs natively) or NVFP4-style 1x16 blocks.
"""
from __future__ import annotations

from typing import Iterable, List, Optional

FP4_RECIPES = ("mxfp4", "nvfp4")


def fp4_default_layers(num_layers: int, recipe: str) -> List[int]:
    """1-indexed layers that run in FP4 when no fp4_layers list is given."""
    if recipe not in FP4_RECIPES:
        raise ValueError(f"unknown FP4 recipe {recipe!r} (expected one of {FP4_RECIPES})")
    if recipe == "mxfp4":
        return list(range(1, num_layers + 1))
    return list(range(2, num_layers))          # nvfp4: first and last layer in BF16


def _check_list(name: str, layers: Optional[Iterable[int]], num_layers: int) -> Optional[List[int]]:
    if layers is None:
        return None
    out = [int(x) for x in layers]
    for x in out:
        if x < 1 or x > num_layers:
            raise ValueError(f"{name}: layer {x} outside 1..{num_layers}")
    if len(set(out)) != len(out):
        raise ValueError(f"{name}: repeated layer numbers {out}")
    return out


def layer_precisions(num_layers: int, *, fp8_enabled: bool = False, fp4_enabled: bool = False,
                     fp8_layers: Optional[Iterable[int]] = None, fp4_layers: Optional[Iterable[int]] = None,
                     fp4_recipe: str = "mxfp4") -> List[str]:
    """Precision of each layer, in layer order: "bf16", "mxfp8", or the FP4
    recipe ("mxfp4" / "nvfp4")."""
    if num_layers < 1:
        raise ValueError("num_layers must be at least 1")
    if fp4_recipe not in FP4_RECIPES:
        raise ValueError(f"unknown FP4 recipe {fp4_recipe!r} (expected one of {FP4_RECIPES})")
    l8 = _check_list("fp8_layers", fp8_layers, num_layers)
    l4 = _check_list("fp4_layers", fp4_layers, num_layers)
    if l8 is not None and not fp8_enabled:
        raise ValueError("fp8_layers given but FP8 is not enabled")
    if l4 is not None and not fp4_enabled:
        raise ValueError("fp4_layers given but FP4 is not enabled")
    if l8 is not None and l4 is not None and set(l8) & set(l4):
        raise ValueError(f"layers {sorted(set(l8) & set(l4))} are in both fp8_layers and fp4_layers")
    every = set(range(1, num_layers + 1))
    s8: set = set()
    s4: set = set()
    if fp8_enabled and fp4_enabled:
        if l8 is not None and l4 is not None:
            s8, s4 = set(l8), set(l4)
        elif l8 is not None:
            s8 = set(l8)
            s4 = every - s8
        elif l4 is not None:
            s4 = set(l4)
            s8 = every - s4
        else:
            s4 = set(fp4_default_layers(num_layers, fp4_recipe))
            s8 = every - s4
    elif fp8_enabled:
        s8 = set(l8) if l8 is not None else every
    elif fp4_enabled:
        s4 = set(l4) if l4 is not None else set(fp4_default_layers(num_layers, fp4_recipe))
    return ["mxfp8" if i in s8 else (fp4_recipe if i in s4 else "bf16") for i in range(1, num_layers + 1)]

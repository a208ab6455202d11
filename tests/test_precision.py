"""Layer-wise precision selection, pinned to the examples the pages give
("TransformerEngine-accelerated Llama 3 training with native PyTorch training
loop", Layer-Wise Precision; "examples/llama: default-on fusion & DP-comm
perf toggles - #141", Changes: the recipe-aware FP4 default)."""
import pytest

from mxfp8_block_scaled_mx_amd.precision import fp4_default_layers, layer_precisions


def test_both_lists_rest_bf16():
    # layers 1-3 in FP8, 4-6 in FP4, the rest in BF16 on a model of more than 6 layers
    got = layer_precisions(8, fp8_enabled=True, fp4_enabled=True, fp8_layers=[1, 2, 3], fp4_layers=[4, 5, 6])
    assert got == ["mxfp8"] * 3 + ["mxfp4"] * 3 + ["bf16"] * 2


def test_one_list_other_format_claims_the_rest():
    # fp8_layers=[1,2,3] with FP4 enabled and no fp4_layers: layers 4..N in FP4
    got = layer_precisions(10, fp8_enabled=True, fp4_enabled=True, fp8_layers=[1, 2, 3])
    assert got == ["mxfp8"] * 3 + ["mxfp4"] * 7
    got = layer_precisions(5, fp8_enabled=True, fp4_enabled=True, fp4_layers=[2, 4], fp4_recipe="nvfp4")
    assert got == ["mxfp8", "nvfp4", "mxfp8", "nvfp4", "mxfp8"]


def test_recipe_defaults():
    # mxfp4: every layer in FP4; nvfp4: first and last layer kept in BF16
    assert fp4_default_layers(4, "mxfp4") == [1, 2, 3, 4]
    assert fp4_default_layers(4, "nvfp4") == [2, 3]
    assert layer_precisions(6, fp4_enabled=True, fp4_recipe="nvfp4") == ["bf16"] + ["nvfp4"] * 4 + ["bf16"]
    assert layer_precisions(3, fp4_enabled=True) == ["mxfp4"] * 3
    # both enabled, no lists (reading): the FP4 default layers, FP8 takes the rest
    assert layer_precisions(4, fp8_enabled=True, fp4_enabled=True, fp4_recipe="nvfp4") == \
        ["mxfp8", "nvfp4", "nvfp4", "mxfp8"]


def test_single_format_and_none():
    assert layer_precisions(3, fp8_enabled=True) == ["mxfp8"] * 3
    assert layer_precisions(4, fp8_enabled=True, fp8_layers=[2]) == ["bf16", "mxfp8", "bf16", "bf16"]
    assert layer_precisions(2) == ["bf16", "bf16"]
    assert layer_precisions(1, fp4_enabled=True, fp4_recipe="nvfp4") == ["bf16"]


@pytest.mark.parametrize("kw", [
    dict(fp8_layers=[1]),                                           # FP8 not enabled
    dict(fp8_enabled=True, fp8_layers=[0]),                         # 1-indexed
    dict(fp8_enabled=True, fp8_layers=[5]),                         # past the last layer
    dict(fp8_enabled=True, fp8_layers=[1, 1]),
    dict(fp8_enabled=True, fp4_enabled=True, fp8_layers=[1, 2], fp4_layers=[2, 3]),
    dict(fp4_enabled=True, fp4_recipe="fp4"),
])
def test_rejected(kw):
    with pytest.raises(ValueError):
        layer_precisions(4, **kw)

"""How much of the bf16 parity budget the bf16 activation recipe consumes by
itself, with no kernel involved (tests/bf16_recipe.py applies only the
recipe's roundings to the oracle's float64 arithmetic).

On the 31-token LeVJEPA-style clip (CLS + 5 x 3 x 2 patches, ViT-L width) the
recipe alone reaches, against the exact oracle: max-abs 0.0124 after 2
layers, 0.0178 after 4, 0.0182 after 6 and 0.0149 after 8 (the max over
31 x 1024 features fluctuates with depth), with per-token cosines above
0.99998.  The small-clip bf16 GPU test therefore runs 4 layers: the recipe
then leaves the kernels about a tenth of the 2e-2 max-abs gate, and deeper
clips would mostly measure the recipe.  The full-depth bf16 workloads are
checked against stored oracle samples, where many more tokens average the
per-feature extremes."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

import bf16_recipe as R
from gpu_util import ABS_BF16, COS_BF16, abs_gate

# expected max-abs of the recipe alone, per depth (see the module docstring)
EXPECTED = {2: 0.0124, 4: 0.0178, 6: 0.0182, 8: 0.0149}


@pytest.fixture(scope="module")
def clip():
    cfg = W.CONFIGS[4].replace(frames=5, height=48, width=32, n_layer=8)
    return cfg, W.make_workload(cfg)


def test_rounding_helper():
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -7 + 2.0 ** -9])
    assert list(R.bf16(x)) == [1.0, 1.0 + 2.0 ** -6, -2.5, 1.0 + 2.0 ** -7]


@pytest.mark.parametrize("layers", sorted(EXPECTED))
def test_recipe_error_by_depth(clip, layers):
    cfg, wl = clip
    ref, _ = oracle.encoder_forward(cfg, wl.weights, wl.pixels, n_layers=layers)
    emu = R.encoder_forward_recipe(cfg, wl.weights, wl.pixels, n_layers=layers)
    st = oracle.compare(emu, ref)
    print(layers, st)
    assert st["min_cos"] >= 1 - 2e-5
    assert abs(st["maxabs"] - EXPECTED[layers]) <= 1e-4, st["maxabs"]
    # the depth the GPU test runs leaves the kernels some room under the gate
    if layers == 4:
        assert st["maxabs"] < ABS_BF16 and st["min_cos"] > COS_BF16


def test_recipe_error_at_vit_g_depth():
    """The 40-layer ViT-g forward: the recipe alone reaches max-abs 0.0200 on
    a 4-frame 128 x 128 clip (128 tokens), at the 2e-2 gate of the 24-layer
    workloads; the full 18432-token clip takes the max over 144 times as many
    tokens.  Its gate (abs_gate(40)) leaves the kernels 30 % of it."""
    cfg = W.CONFIGS[3].replace(frames=4, height=128, width=128)
    assert cfg.n_layer == 40 and cfg.n_tokens == 128
    wl = W.make_workload(cfg)
    ref, _ = oracle.encoder_forward(cfg, wl.weights, wl.pixels)
    emu = R.encoder_forward_recipe(cfg, wl.weights, wl.pixels)
    st = oracle.compare(emu, ref)
    print(st)
    assert st["min_cos"] >= 1 - 2e-5
    assert abs(st["maxabs"] - 0.0200) <= 1e-4, st["maxabs"]
    assert st["maxabs"] >= 0.95 * ABS_BF16
    assert st["maxabs"] <= 0.7 * abs_gate(cfg.n_layer)

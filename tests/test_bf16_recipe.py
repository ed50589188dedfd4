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


@pytest.mark.parametrize("name", ["vjepa2", "vjepa21", "levjepa"])
def test_sensitised_bf16_gate_sees_planted_mistakes(name):
    """On the sensitised small clips in bf16 (4 layers) the recipe alone is
    0.03-0.16 max-abs from the oracle; the GPU test of those clips allows
    twice that.  A wrong RoPE layout, a missing interpolation or a full mask
    in place of the block-causal one moves the oracle's output at least five
    times further than that allowance in max-abs (19-57 times the recipe's
    own distance) and a hundred times further in per-token cosine."""
    small = {
        "vjepa2": W.CONFIGS[2].replace(frames=4, height=48, width=64, batch=2),
        "vjepa21": W.CONFIGS[3].replace(frames=4, height=64, width=48),
        "levjepa": W.CONFIGS[4].replace(frames=5, height=48, width=32),
    }
    cfg = W.sensitised(small[name].replace(n_layer=4), std_qk=0.1, std_tok=1.0)
    wl = W.make_workload(cfg)
    ref, _ = oracle.encoder_forward(cfg, wl.weights, wl.pixels)
    emu = R.encoder_forward_recipe(cfg, wl.weights, wl.pixels)
    st = oracle.compare(emu, ref)
    allow_abs, allow_cos = 2.0 * st["maxabs"] + 2e-3, 2.0 * (1.0 - st["min_cos"]) + 1e-6
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)

    def run(c, pos, visible):
        Z = oracle.embed(c, wl.weights, wl.pixels)
        for blk in wl.weights.blocks:
            Z = oracle.encoder_block(Z, blk, c, pos, visible)
        return oracle.layer_norm(Z, wl.weights.norm_w, wl.weights.norm_b, c.ln_eps)

    planted = [run(cfg.replace(rope_layout=1 - cfg.rope_layout), rp, vis)]
    if cfg.rope_interpolate:
        planted.append(run(cfg, oracle.rope_and_mask(cfg.replace(rope_interpolate=0), wl.pixels.shape)[0], vis))
    if cfg.attn_mode == W.ATTN_BLOCK_CAUSAL:
        planted.append(run(cfg, rp, oracle.rope_and_mask(cfg.replace(attn_mode=W.ATTN_FULL), wl.pixels.shape)[1]))
    for bad in planted:
        sb = oracle.compare(bad, ref)
        assert sb["maxabs"] > 5 * allow_abs and 1.0 - sb["min_cos"] > 100 * allow_cos, (sb, st)

"""Pins of the V-JEPA 2.1 encoder options of the oracle (jepa.cpp "GGUF
schema (v1)": a separate 1x16x16 image tokenizer with its own modality
vector, and one norm per hierarchical layer): torch's convolutions and
layer_norm in float64, and closed forms."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

torch = pytest.importorskip("torch")
F = torch.nn.functional

TINY = W.CONFIGS[3].replace(name="tiny_vjepa21", embed_dim=48, n_head=2, ffn_dim=64, n_layer=4, patch_size=4,
                            frames=4, height=8, width=12, batch=2, dtype=W.DTYPE_F32, rope_ref_grid=4,
                            image_patch_embed=1, hier_layers=(0, 2, 3), std_tok=1.0)


def test_image_goes_through_the_image_tokenizer():
    cfg = TINY.replace(frames=1)
    wl = W.make_workload(cfg)
    w = wl.weights
    assert cfg.grid == (1, 2, 3) and w.patch_img_w.shape == (48, 3 * 4 * 4)
    Z = oracle.embed(cfg, w, wl.pixels)
    x = torch.from_numpy(wl.pixels[:, :, 0].astype(np.float64))
    k = torch.from_numpy(w.patch_img_w.astype(np.float64)).reshape(48, 3, 4, 4)
    conv = F.conv2d(x, k, torch.from_numpy(w.patch_img_b.astype(np.float64)), stride=4)
    ref = conv.flatten(2).transpose(1, 2).numpy() + w.mod_img.astype(np.float64)
    assert np.abs(Z - ref).max() < 1e-12


def test_video_keeps_the_tubelet_tokenizer():
    wl = W.make_workload(TINY)
    w = wl.weights
    Z = oracle.embed(TINY, w, wl.pixels)
    x = torch.from_numpy(wl.pixels.astype(np.float64))
    k = torch.from_numpy(w.patch_w.astype(np.float64)).reshape(48, 3, 2, 4, 4)
    conv = F.conv3d(x, k, torch.from_numpy(w.patch_b.astype(np.float64)), stride=(2, 4, 4))
    ref = conv.flatten(2).transpose(1, 2).numpy() + w.mod.astype(np.float64)
    assert np.abs(Z - ref).max() < 1e-12


@pytest.mark.parametrize("frames", [1, 4])
def test_hierarchical_outputs(frames):
    """Output k is block hier_layers[k]'s residual stream through norm k
    (torch's layer_norm on the residual of a forward stopped after that
    block); the final output does not depend on the hierarchical norms."""
    cfg = TINY.replace(frames=frames)
    wl = W.make_workload(cfg)
    out, pooled, hier = oracle.encoder_forward(cfg, wl.weights, wl.pixels, return_hier=True)
    assert hier.shape == (3,) + out.shape
    for k, l in enumerate(cfg.hier_layers):
        _, _, Z = oracle.encoder_forward(cfg, wl.weights, wl.pixels, n_layers=l + 1, return_residual=True)
        ref = F.layer_norm(torch.from_numpy(Z), (48,), torch.from_numpy(wl.weights.hier_norm_w[k].astype(np.float64)),
                           torch.from_numpy(wl.weights.hier_norm_b[k].astype(np.float64)), cfg.ln_eps).numpy()
        assert np.abs(hier[k] - ref).max() < 1e-12
    w2 = W.make_workload(cfg).weights
    w2.hier_norm_w = [x * 3.0 for x in w2.hier_norm_w]
    out2, _, _ = oracle.encoder_forward(cfg, w2, wl.pixels, return_hier=True)
    assert np.array_equal(out, out2)

"""Sensitised negative controls, on the CPU oracle only.

With N(0, 0.02) weights the attention is close to uniform and several wrong
readings of the pages would still pass the bf16 gates.  The sensitised
variants (large q/k rows, large CLS / modality vectors) make them visible:
each planted mistake below must FAIL the gate against the correct oracle,
the way the pages require an unmasked control to disagree and a +1 % weight
perturbation to fail (jepa.cpp "Architecture", section "Testing and parity
methodology").  Mistakes are planted by handing the oracle wrong positions /
masks / inputs; the oracle's code itself is unchanged."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

GATE_COS, GATE_ABS = 0.9999, 2e-2


def _fails_gate(a, b):
    st = oracle.compare(a, b)
    return st["min_cos"] < GATE_COS or st["maxabs"] > GATE_ABS


def _run(cfg, w, pixels, rope_pos, visible, embed_fn=None):
    Z = oracle.embed(cfg, w, pixels) if embed_fn is None else embed_fn()
    for blk in w.blocks:
        Z = oracle.encoder_block(Z, blk, cfg, rope_pos, visible)
    return oracle.layer_norm(Z, w.norm_w, w.norm_b, cfg.ln_eps)


def _small(cfg, **kw):
    """Shrink a config's clip and depth, keep its head_dim, families and mask."""
    return W.sensitised(cfg.replace(n_layer=2, embed_dim=256, n_head=4, ffn_dim=512, dtype=W.DTYPE_F32,
                                    batch=1, **kw))


@pytest.fixture(scope="module")
def vjepa2():
    cfg = _small(W.CONFIGS[2], frames=4, height=64, width=64)
    return cfg, W.make_workload(cfg)


@pytest.fixture(scope="module")
def vjepa21():
    cfg = _small(W.CONFIGS[3], frames=4, height=96, width=96)
    return cfg, W.make_workload(cfg)


@pytest.fixture(scope="module")
def levjepa():
    cfg = _small(W.CONFIGS[4], frames=4, height=64, width=64)
    return cfg, W.make_workload(cfg)


def test_wrong_rope_layout_fails(vjepa2):
    cfg, wl = vjepa2
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    bad = _run(cfg.replace(rope_layout=W.LAYOUT_INTERLEAVED), wl.weights, wl.pixels, rp, vis)
    assert _fails_gate(bad, good)


def test_missing_interpolate_fails(vjepa21):
    cfg, wl = vjepa21
    assert cfg.grid[1] != cfg.rope_ref_grid
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    rp_bad, _ = oracle.rope_and_mask(cfg.replace(rope_interpolate=0), wl.pixels.shape)
    assert _fails_gate(_run(cfg, wl.weights, wl.pixels, rp_bad, vis), good)


def test_interpolating_time_axis_fails(vjepa21):
    cfg, wl = vjepa21
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    gt = cfg.grid[0]
    s = oracle.rope_interpolate_scale(cfg.rope_ref_grid, gt)
    bad_pos = [rp[0] * s, rp[1], rp[2]]
    assert _fails_gate(_run(cfg, wl.weights, wl.pixels, bad_pos, vis), good)


def test_dropped_modality_vector_fails(vjepa21):
    cfg, wl = vjepa21
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    bad = _run(cfg.replace(modality_embed=0), wl.weights, wl.pixels, rp, vis)
    assert _fails_gate(bad, good)


def test_off_by_one_frame_id_fails(levjepa):
    cfg, wl = levjepa
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    S = cfg.grid[1] * cfg.grid[2]
    # frame ids computed without removing the CLS prefix: (id) // S
    N = cfg.n_tokens
    f = np.arange(N) // S
    bad_vis = (f[:, None] >= f[None, :]) & (np.arange(N)[None, :] >= 1)
    bad_vis[0] = True
    assert _fails_gate(_run(cfg, wl.weights, wl.pixels, rp, bad_vis), good)


def test_open_cls_column_fails(levjepa):
    cfg, wl = levjepa
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    bad_vis = vis.copy()
    bad_vis[:, 0] = True
    assert _fails_gate(_run(cfg, wl.weights, wl.pixels, rp, bad_vis), good)


def test_unmasked_control_fails(levjepa):
    cfg, wl = levjepa
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    assert _fails_gate(_run(cfg, wl.weights, wl.pixels, rp, None), good)


def test_rotated_cls_fails(levjepa):
    """Treating the CLS as a patch at grid position (0,0,0) and shifting all
    patch ids by one (ids counted from the CLS) must fail."""
    cfg, wl = levjepa
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    t, h, w = oracle.token_grid_positions(cfg.n_tokens, cfg.grid)
    bad_pos = [t[1:], h[1:], w[1:]]
    assert _fails_gate(_run(cfg, wl.weights, wl.pixels, bad_pos, vis), good)


def test_weight_perturbation_of_one_percent_fails(vjepa2):
    cfg, wl = vjepa2
    rp, vis = oracle.rope_and_mask(cfg, wl.pixels.shape)
    good = _run(cfg, wl.weights, wl.pixels, rp, vis)
    blk = wl.weights.blocks[0]
    keep = blk.up_w
    blk.up_w = keep * np.float32(1.01)
    try:
        bad = _run(cfg, wl.weights, wl.pixels, rp, vis)
    finally:
        blk.up_w = keep
    st = oracle.compare(bad, good)
    assert st["rel"] > 1e-4       # the fp32 gate catches it

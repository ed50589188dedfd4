"""Pins of the predictor oracle (oracle/predictor.py) against closed forms and
invariants that do not reuse its own code path."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

TINY = W.PredictorConfig("tiny_predictor", embed_dim=48, enc_dim=40, n_layer=2, n_head=3, ffn_dim=96,
                         n_mask_tokens=3, grid=(3, 4, 5), batch=2, n_ctx=25, n_tgt=20, dtype=W.DTYPE_F32,
                         std_w=0.1, std_tok=0.5, seed=7)


def _wl(cfg):
    return W.make_predictor_workload(cfg)


def test_id_positions_follow_the_token_order():
    grid = (3, 4, 5)
    t, h, w = oracle.id_positions(np.arange(60), grid)
    tt, hh, ww = oracle.token_grid_positions(60, grid)
    assert np.array_equal(t, tt) and np.array_equal(h, hh) and np.array_equal(w, ww)
    # a token id is t*gh*gw + h*gw + w
    assert np.array_equal(t * 20 + h * 5 + w, np.arange(60))


def test_zero_layers_gives_projected_mask_token():
    """With no blocks every target is proj(LN(mask token)), whatever its
    position or the context: pins the mask-token choice, the restore of the
    input order and the output projection."""
    wl = _wl(TINY)
    hp = TINY.hparams()
    w = wl.weights
    for mi in range(TINY.n_mask_tokens):
        out = oracle.predictor_forward(hp, w, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids, mask_index=mi, n_layers=0)
        m = w.mask_tokens[mi].astype(np.float64)
        y = (m - m.mean()) / np.sqrt(m.var() + TINY.ln_eps)
        expect = y @ w.proj_w.astype(np.float64).T + w.proj_b
        assert np.abs(out - expect[None, None, :]).max() < 1e-12


def test_input_order_does_not_matter():
    """Shuffling the order of the context (with its ids) and of the targets
    permutes nothing but the target outputs accordingly."""
    wl = _wl(TINY)
    hp = TINY.hparams()
    ref = oracle.predictor_forward(hp, wl.weights, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids)
    rng = np.random.default_rng(3)
    pc = np.stack([rng.permutation(TINY.n_ctx) for _ in range(TINY.batch)])
    pt = np.stack([rng.permutation(TINY.n_tgt) for _ in range(TINY.batch)])
    ctx = np.take_along_axis(wl.ctx_ids, pc, axis=1)
    tgt = np.take_along_axis(wl.tgt_ids, pt, axis=1)
    out = oracle.predictor_forward(hp, wl.weights, wl.enc_tokens, ctx, tgt)
    for b in range(TINY.batch):
        assert np.abs(out[b] - ref[b, pt[b]]).max() < 1e-12


def _shift_case(cfg, seed=11):
    """ids kept in frames 0 .. gt-2 (so that one frame later stays on the
    grid) and the encoder features copied to the shifted context ids"""
    wl = _wl(cfg)
    S = cfg.grid[1] * cfg.grid[2]
    rng = np.random.default_rng(seed)
    ctx, tgt = [], []
    for _ in range(cfg.batch):
        perm = rng.permutation((cfg.grid[0] - 1) * S)
        ctx.append(np.sort(perm[:cfg.n_ctx]))
        tgt.append(np.sort(perm[cfg.n_ctx:cfg.n_ctx + cfg.n_tgt]))
    ctx, tgt = np.stack(ctx), np.stack(tgt)
    enc2 = wl.enc_tokens.copy()
    for b in range(cfg.batch):
        enc2[b, ctx[b] + S] = wl.enc_tokens[b, ctx[b]]
    hp = cfg.hparams()
    a = oracle.predictor_forward(hp, wl.weights, wl.enc_tokens, ctx, tgt)
    shifted = oracle.predictor_forward(hp, wl.weights, enc2, ctx + S, tgt + S)
    return a, shifted


def test_uniform_shift_of_positions_is_invisible_with_interleaved_rope():
    """Textbook (interleaved) RoPE makes q.k depend on position differences
    only and the predictor has no absolute position input, so moving every
    token one frame later changes no output (up to rounding)."""
    a, shifted = _shift_case(TINY.replace(rope_layout=W.LAYOUT_INTERLEAVED, n_ctx=12, n_tgt=10))
    assert np.abs(a - shifted).max() < 1e-9 * max(1.0, np.abs(a).max())


def test_tiled_rope_is_not_shift_invariant():
    """Control for the test above: the tiled layout's odd members use other
    frequencies than the even ones (at head_dim 16 here: d = 4 per axis), so
    the same shift does change the output."""
    a, shifted = _shift_case(TINY.replace(n_ctx=12, n_tgt=10))
    assert np.abs(a - shifted).max() > 1e-6


def test_targets_see_the_context():
    wl = _wl(TINY)
    hp = TINY.hparams()
    a = oracle.predictor_forward(hp, wl.weights, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids)
    enc2 = wl.enc_tokens.copy()
    enc2[:, wl.ctx_ids[0, 0]] += 1.0
    b = oracle.predictor_forward(hp, wl.weights, enc2, wl.ctx_ids, wl.tgt_ids)
    assert np.abs(a[0] - b[0]).max() > 1e-6


def test_predictor_rope_head_width_32_uses_ten_dims_per_axis():
    """The predictor's head width 32 gives d = 10 rotated dims per axis (the
    odd-length tiled case the pages single out)."""
    assert W.PREDICTOR.head_dim == 32
    assert oracle.rope_rotated_dims(W.PREDICTOR.head_dim) == 10

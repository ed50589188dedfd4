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


# ---------------------------------------------------------------------------
# V-JEPA 2.1 options: the hierarchical embed MLP, modality vectors, the
# context projection and an output width other than the encoder's
# ---------------------------------------------------------------------------
TINY21 = TINY.replace(name="tiny_predictor_21", n_hier_in=3, embed_hidden=56, out_dim=36, modality_embed=1,
                      context_proj=1, rope_layout=W.LAYOUT_INTERLEAVED, seed=9)


def _ln(x, eps):
    x = np.asarray(x, np.float64)
    m = x.mean(axis=-1, keepdims=True)
    v = ((x - m) ** 2).mean(axis=-1, keepdims=True)
    return (x - m) / np.sqrt(v + eps)


def _gelu(x):
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def test_21_zero_layers_closed_form():
    """With no blocks: each target is proj(LN(mask + mod_video)) and each
    context row proj_ctx(LN(embed2(GELU(embed1([h0; h1; h2])) ) + mod_video)),
    in the order of the id lists (LN gamma 1, beta 0); computed here from the
    definitions, not from the oracle's steps."""
    wl = _wl(TINY21)
    w, hp = wl.weights, TINY21.hparams()
    out, ctx = oracle.predictor_forward(hp, w, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids, mask_index=2, n_layers=0,
                                        return_context=True)
    f64 = lambda a: np.asarray(a, np.float64)
    mod = f64(w.mod_video)
    t = _ln(f64(w.mask_tokens[2]) + mod, TINY21.ln_eps) @ f64(w.proj_w).T + f64(w.proj_b)
    assert out.shape == (TINY21.batch, TINY21.n_tgt, 36)
    assert np.abs(out - t[None, None]).max() < 1e-12
    for b in range(TINY21.batch):
        feats = np.concatenate([f64(wl.enc_tokens[lv, b, wl.ctx_ids[b]]) for lv in range(3)], axis=1)
        h = _gelu(feats @ f64(w.embed_w).T + f64(w.embed_b))
        x = h @ f64(w.embed2_w).T + f64(w.embed2_b) + mod
        c = _ln(x, TINY21.ln_eps) @ f64(w.proj_ctx_w).T + f64(w.proj_ctx_b)
        assert np.abs(ctx[b] - c).max() < 1e-11


def test_21_embed_mlp_is_torch_sequential():
    """The 2-layer embed MLP equals torch's Linear -> GELU (erf) -> Linear in
    float64 on the concatenated levels (checked through the zero-layer
    context rows, whose only other steps are the modality add, LN and the
    context projection)."""
    import torch
    wl = _wl(TINY21)
    w, hp = wl.weights, TINY21.hparams()
    _, ctx = oracle.predictor_forward(hp, w, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids, n_layers=0,
                                      return_context=True)
    mlp = torch.nn.Sequential(torch.nn.Linear(3 * TINY21.enc_dim, 56), torch.nn.GELU(),
                              torch.nn.Linear(56, TINY21.embed_dim)).double()
    with torch.no_grad():
        mlp[0].weight.copy_(torch.from_numpy(np.asarray(w.embed_w, np.float64)))
        mlp[0].bias.copy_(torch.from_numpy(np.asarray(w.embed_b, np.float64)))
        mlp[2].weight.copy_(torch.from_numpy(np.asarray(w.embed2_w, np.float64)))
        mlp[2].bias.copy_(torch.from_numpy(np.asarray(w.embed2_b, np.float64)))
        ln = torch.nn.LayerNorm(TINY21.embed_dim, eps=TINY21.ln_eps, elementwise_affine=False).double()
        b = 1
        feats = torch.cat([torch.from_numpy(np.asarray(wl.enc_tokens[lv, b, wl.ctx_ids[b]], np.float64))
                           for lv in range(3)], dim=1)
        x = ln(mlp(feats) + torch.from_numpy(np.asarray(w.mod_video, np.float64)))
        c = x @ torch.from_numpy(np.asarray(w.proj_ctx_w, np.float64)).T + torch.from_numpy(
            np.asarray(w.proj_ctx_b, np.float64))
    assert np.abs(ctx[b] - c.numpy()).max() < 1e-11


def test_21_level_order_matches_weight_columns():
    """Permuting the hierarchical levels together with the column blocks of
    embed.0 leaves the prediction unchanged; permuting the levels alone does
    not (the levels are concatenated in order)."""
    wl = _wl(TINY21)
    w, hp = wl.weights, TINY21.hparams()
    ref = oracle.predictor_forward(hp, w, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids)
    perm = [2, 0, 1]
    De = TINY21.enc_dim
    enc_p = wl.enc_tokens[perm]
    import copy
    w2 = copy.copy(w)
    w2.embed_w = np.concatenate([w.embed_w[:, lv * De:(lv + 1) * De] for lv in perm], axis=1)
    same = oracle.predictor_forward(hp, w2, enc_p, wl.ctx_ids, wl.tgt_ids)
    assert np.abs(same - ref).max() < 1e-12
    other = oracle.predictor_forward(hp, w, enc_p, wl.ctx_ids, wl.tgt_ids)
    assert np.abs(other - ref).max() > 1e-3


def test_21_modality_vector_follows_the_grid():
    """A one-frame grid takes the image vector, a clip the video vector; the
    vector reaches every token (a constant added to all tokens before the
    first LayerNorm is not removed by it: LN subtracts the row mean, not a
    shared vector)."""
    cfg = TINY21.replace(grid=(1, 6, 7), n_ctx=20, n_tgt=15)
    wl = _wl(cfg)
    w, hp = wl.weights, cfg.hparams()
    ref = oracle.predictor_forward(hp, w, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids)
    import copy
    w2 = copy.copy(w)
    w2.mod_video = w.mod_video + np.linspace(-1.0, 1.0, w.mod_video.size, dtype=np.float32)  # unused here
    assert np.abs(oracle.predictor_forward(hp, w2, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids) - ref).max() == 0.0
    w3 = copy.copy(w)
    # a non-uniform change (LayerNorm removes a shift shared by every feature)
    w3.mod_img = w.mod_img + np.random.default_rng(1).normal(0.0, 0.5, w.mod_img.shape).astype(np.float32)
    assert np.abs(oracle.predictor_forward(hp, w3, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids) - ref).max() > 1e-3


def test_21_context_rows_follow_ctx_ids():
    """Shuffling the context id list permutes the projected context rows the
    same way and leaves the targets unchanged."""
    wl = _wl(TINY21)
    w, hp = wl.weights, TINY21.hparams()
    out, ctx = oracle.predictor_forward(hp, w, wl.enc_tokens, wl.ctx_ids, wl.tgt_ids, return_context=True)
    rng = np.random.default_rng(5)
    pc = np.stack([rng.permutation(TINY21.n_ctx) for _ in range(TINY21.batch)])
    ids = np.take_along_axis(wl.ctx_ids, pc, axis=1)
    out2, ctx2 = oracle.predictor_forward(hp, w, wl.enc_tokens, ids, wl.tgt_ids, return_context=True)
    assert np.abs(out2 - out).max() < 1e-12
    for b in range(TINY21.batch):
        assert np.abs(ctx2[b] - ctx[b, pc[b]]).max() < 1e-12


def test_21_options_off_draw_the_vjepa2_workload():
    """A configuration without the 2.1 options draws exactly the V-JEPA 2
    workload (the options' tensors are drawn after everything else)."""
    a = _wl(TINY)
    b = _wl(TINY.replace(out_dim=TINY.enc_dim))
    assert np.array_equal(a.enc_tokens, b.enc_tokens) and np.array_equal(a.weights.proj_w, b.weights.proj_w)
    assert a.weights.embed2_w is None and a.weights.mod_img is None and a.weights.proj_ctx_w is None

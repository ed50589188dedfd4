"""CPU oracle of the masked-latent predictor that follows the encoder (numpy
float64).

TEST INFRASTRUCTURE ONLY, like oracle/encoder.py: imported by the test suite
and the benchmark's CPU-baseline leg, never by the library.

The steps follow SkyVision.cpp README, V-JEPA 2 backend notes ("masked-latent
predictor"): take the encoder features at the context token ids, project them
to the predictor width, append one mask token per target id, put all tokens in
position order, run the predictor's own pre-LN blocks with 3-D RoPE on those
positions, normalise, restore the input order, keep the target rows and project
them back to the encoder width.  The hyperparameters are those of jepa.cpp "GGUF
schema (v1)", section "Predictor (jepa.pred.*)": its own width, depth, heads and
ffn, n_mask_tokens learned tokens, and its own RoPE convention on the fixed token
grid (no interpolation).

Readings:
  * the blocks are the encoder's block (pre-LN, fused [q; k; v], GELU-erf,
    residuals), with full attention over context and target tokens and no
    prefix token;
  * RoPE positions of a token id are its (t, h, w) on the grid, decoded in the
    encoder's token order (t, then h, then w);
  * which of the n_mask_tokens tokens fills the targets is a parameter
    (mask_index): the pages note that the reference always uses index 1;
  * ids are distinct within an item (context and targets are disjoint), so the
    position order is unique.

V-JEPA 2.1 options ("GGUF schema (v1)", "Predictor (jepa.pred.*)": n_hier_in,
modality_embed, context_proj, out_dim; tensors pred.embed.0 / .2,
pred.mod_embed_img / _video, pred.proj_context), with these readings:
  * n_hier_in > 1: a context token's input is the concatenation, in level
    order, of its n_hier_in hierarchical encoder features, and pred.embed is
    the 2-layer MLP embed.0 -> GELU (erf) -> embed.2 (the .0 / .2 names are
    the layers around the activation of a sequential MLP; the pages name no
    activation there, GELU-erf is the one every MLP of the family uses);
  * the modality vector (image for a one-frame grid, video otherwise, as the
    encoder picks its tokenizer) is added to every predictor token, context
    and mask tokens alike, before the blocks;
  * pred.proj maps to out_dim (the teacher's width in 2.1, the encoder's in
    V-JEPA 2), and pred.proj_context maps the context rows of the final norm's
    output to the same width (the context half of "return all tokens"),
    returned in the order of ctx_ids.
"""
from __future__ import annotations

import numpy as np

from . import encoder as E


def id_positions(ids: np.ndarray, grid):
    """Patch token id -> (t, h, w) on the grid (encoder token order)."""
    gt, gh, gw = grid
    ids = np.asarray(ids, dtype=np.int64)
    t = ids // (gh * gw)
    h = (ids % (gh * gw)) // gw
    w = ids % gw
    return t.astype(np.float64), h.astype(np.float64), w.astype(np.float64)


def _block_hp(hp):
    return dict(n_head=hp["n_head"], ln_eps=hp["ln_eps"], cls_token=0, rope=1, rope_layout=hp["rope_layout"],
                rope_theta=hp["rope_theta"])


def predictor_forward(hp, w, enc_tokens, ctx_ids, tgt_ids, mask_index=1, n_layers=None, return_context=False):
    """enc_tokens [B, N_grid, enc_dim] (with n_hier_in > 1: [n_hier_in, B,
    N_grid, enc_dim]); ctx_ids [B, n_ctx]; tgt_ids [B, n_tgt] -> predicted
    target features [B, n_tgt, out_dim] (float64); with return_context also
    the projected context rows [B, n_ctx, out_dim] (needs context_proj)."""
    n_hier = int(hp.get("n_hier_in", 1) or 1)
    enc = np.asarray(enc_tokens)
    if n_hier == 1 and enc.ndim == 4:
        enc = enc[0]
    B = enc.shape[-3]
    n_ctx, n_tgt = ctx_ids.shape[1], tgt_ids.shape[1]
    bhp = _block_hp(hp)
    L = len(w.blocks) if n_layers is None else n_layers
    out_dim = int(hp.get("out_dim", 0) or hp["enc_dim"])
    mod = None
    if hp.get("modality_embed", 0):
        mod = E._f64(w.mod_img if hp["grid"][0] == 1 else w.mod_video)
    out = np.empty((B, n_tgt, out_dim))
    out_ctx = np.empty((B, n_ctx, out_dim)) if return_context else None
    for b in range(B):
        if n_hier > 1:
            feats = np.concatenate([enc[lv, b, ctx_ids[b]] for lv in range(n_hier)], axis=1)
            x_ctx = E.linear(E.gelu_erf(E.linear(feats, w.embed_w, w.embed_b)), w.embed2_w, w.embed2_b)
        else:
            x_ctx = E.linear(enc[b, ctx_ids[b]], w.embed_w, w.embed_b)
        x_tgt = np.repeat(E._f64(w.mask_tokens[mask_index])[None, :], n_tgt, axis=0)
        if mod is not None:
            x_ctx = x_ctx + mod
            x_tgt = x_tgt + mod
        ids = np.concatenate([ctx_ids[b], tgt_ids[b]]).astype(np.int64)
        x = np.concatenate([x_ctx, x_tgt], axis=0)
        assert len(np.unique(ids)) == len(ids), "token ids must be distinct"
        order = np.argsort(ids, kind="stable")
        x = x[order][None]
        pos = id_positions(ids[order], hp["grid"])
        for blk in w.blocks[:L]:
            x = E.encoder_block(x, blk, bhp, pos, None)
        x = E.layer_norm(x[0], w.norm_w, w.norm_b, hp["ln_eps"])
        back = np.empty_like(order)
        back[order] = np.arange(len(order))
        x = x[back]
        out[b] = E.linear(x[n_ctx:], w.proj_w, w.proj_b)
        if return_context:
            out_ctx[b] = E.linear(x[:n_ctx], w.proj_ctx_w, w.proj_ctx_b)
    return (out, out_ctx) if return_context else out

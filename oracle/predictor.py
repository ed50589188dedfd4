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


def predictor_forward(hp, w, enc_tokens, ctx_ids, tgt_ids, mask_index=1, n_layers=None):
    """enc_tokens [B, N_grid, enc_dim]; ctx_ids [B, n_ctx]; tgt_ids [B, n_tgt]
    -> predicted target features [B, n_tgt, enc_dim] (float64)."""
    B = enc_tokens.shape[0]
    n_ctx, n_tgt = ctx_ids.shape[1], tgt_ids.shape[1]
    bhp = _block_hp(hp)
    L = len(w.blocks) if n_layers is None else n_layers
    out = np.empty((B, n_tgt, hp["enc_dim"]))
    for b in range(B):
        x_ctx = E.linear(enc_tokens[b, ctx_ids[b]], w.embed_w, w.embed_b)
        x_tgt = np.repeat(E._f64(w.mask_tokens[mask_index])[None, :], n_tgt, axis=0)
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
        out[b] = E.linear(x[back][n_ctx:], w.proj_w, w.proj_b)
    return out

"""CPU oracle of the attentive-pool head and its classifier (numpy float64).

TEST INFRASTRUCTURE ONLY, like oracle/encoder.py: imported by the test suite
and the benchmark's CPU-baseline leg, never by the library.

The head of jepa.cpp "GGUF schema (v1)", section "Head (jepa.head.*)", kind
attentive_pool, as SkyVision.cpp README, V-JEPA 2 backend notes, describes the
pooler and classifier heads:

  1. n_pool_layers ordinary pre-LN self-attention blocks (the encoder block's
     layout, no RoPE, no mask) over the whole token stream;
  2. one learned query token attends over all tokens: keys and values come
     from a LayerNorm of the tokens (ln_kv); the query itself is not
     normalised; q, k, v are linear maps with biases; multi-head softmax
     attention; the heads are concatenated with NO output projection;
  3. the raw query is the residual of the cross-attention:  y = query + attn;
  4. an MLP with its own LayerNorm (ln2) and a residual:  y += mlp(ln2(y));
  5. the classifier is a linear map on y (no final norm).

Readings:
  * the head's input is the encoder's output (after its final norm), the
    stream the pooler runs on when the pooled feature is the embedding;
  * the MLP is fc1, GELU (erf form, as the encoder's FFN), fc2, and it sits in
    a residual branch like the blocks' FFN;
  * the cross-attention has as many heads as the encoder (embed_dim /
    n_head = head width), scale 1/sqrt(head width);
  * the pooler blocks have no layer-scale.
"""
from __future__ import annotations

import math

import numpy as np

from . import encoder as E


def _block_hp(hp):
    return dict(n_head=hp["n_head"], ln_eps=hp["ln_eps"], cls_token=0, rope=0)


def cross_attention_pool(hp, w, x):
    """Steps 2-4 on x [B, N, D] -> pooled [B, D]."""
    B, N, D = x.shape
    H = hp["n_head"]
    hd = D // H
    kv = E.layer_norm(x, w.ln_kv_w, w.ln_kv_b, hp["ln_eps"])
    q0 = E._f64(w.query)
    q = E.linear(q0[None, :], w.q_w, w.q_b)[0]          # [D]: the same query for every item
    k = E.linear(kv, w.k_w, w.k_b)                       # [B, N, D]
    v = E.linear(kv, w.v_w, w.v_b)
    attn = np.empty((B, D))
    for b in range(B):
        for h in range(H):
            sl = slice(h * hd, (h + 1) * hd)
            attn[b, sl] = E.attention(q[None, sl], k[b, :, sl], v[b, :, sl])[0]
    y = q0[None, :] + attn
    f = E.linear(E.gelu_erf(E.linear(E.layer_norm(y, w.ln2_w, w.ln2_b, hp["ln_eps"]), w.up_w, w.up_b)),
                 w.down_w, w.down_b)
    return y + f


def attentive_pool_forward(hp, w, tokens, n_layers=None):
    """tokens [B, N, D] -> (pooled [B, D], logits [B, n_classes]) in float64."""
    x = E._f64(tokens)
    L = len(w.blocks) if n_layers is None else n_layers
    bhp = _block_hp(hp)
    for blk in w.blocks[:L]:
        x = E.encoder_block(x, blk, bhp, None, None)
    pooled = cross_attention_pool(hp, w, x)
    logits = E.linear(pooled, w.cls_w, w.cls_b)
    return pooled, logits

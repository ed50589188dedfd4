"""A CPU emulation of the bf16 activation recipe (test helper, not a test).

The bf16 path of the library keeps an fp32 residual stream and fp32
accumulation, and rounds to bf16 (round to nearest even) exactly where its
kernels hand a 16-bit operand to the next step:

  pixels          split into hi = bf16(x) and lo = bf16(x - hi) (about 16
                  significant bits reach the patch GEMM)
  LN1 / LN2 out   bf16 (operands of the QKV and up projections)
  q, k, v         bf16 after bias and RoPE (RoPE rotates the fp32 value)
  softmax         the weights exp(s - m) are rounded to bf16 (operands of the
                  P.V product) and the row sum adds the rounded weights
  attention out   bf16 (operand of the out projection)
  GELU out        bf16 (operand of the down projection)

Everything else is the oracle's float64 arithmetic (oracle/encoder.py), so
the difference between this emulation and the oracle is the error of the
recipe itself, with no kernel involved.  The tests use it to show how much
of the bf16 parity budget the recipe alone consumes at a given depth.
"""
from __future__ import annotations

import numpy as np

import oracle


def bf16(x) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest, ties to even) -> fp64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32)
    # NaN / inf pass through unchanged (none occur here)
    out = np.where(np.isfinite(f), out, f)
    return out.astype(np.float64)


def fp32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _attention_rounded(q, k, v, visible):
    """softmax(q k^T / sqrt(hd)) v with the weights rounded to bf16 before the
    product and the normaliser summed over the rounded weights."""
    hd = q.shape[1]
    s = (q @ k.T) / np.sqrt(hd)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    p = bf16(np.exp(s - s.max(axis=1, keepdims=True)))
    return (p @ v) / p.sum(axis=1, keepdims=True)


def _block(Z, blk, hp, rope_pos, visible):
    B, N, D = Z.shape
    H = hp.n_head
    hd = D // H
    p = hp.n_prefix
    Y = bf16(oracle.layer_norm(Z, blk.ln1_w, blk.ln1_b, hp.ln_eps))
    qkv = fp32(oracle.linear(Y, blk.qkv_w, blk.qkv_b))
    q = qkv[..., 0:D].reshape(B, N, H, hd).transpose(0, 2, 1, 3).copy()
    k = qkv[..., D:2 * D].reshape(B, N, H, hd).transpose(0, 2, 1, 3).copy()
    v = qkv[..., 2 * D:3 * D].reshape(B, N, H, hd).transpose(0, 2, 1, 3)
    if rope_pos is not None:
        q[:, :, p:] = oracle.rope3d_apply(q[:, :, p:], rope_pos, hp.rope_layout, hp.rope_theta)
        k[:, :, p:] = oracle.rope3d_apply(k[:, :, p:], rope_pos, hp.rope_layout, hp.rope_theta)
    q, k, v = bf16(q), bf16(k), bf16(v)
    O = np.empty((B, H, N, hd))
    for b in range(B):
        for h in range(H):
            O[b, h] = _attention_rounded(q[b, h], k[b, h], v[b, h], visible)
    O = bf16(O.transpose(0, 2, 1, 3).reshape(B, N, D))
    a = oracle.linear(O, blk.out_w, blk.out_b)
    if blk.ls1 is not None:
        a = a * blk.ls1
    Z = fp32(Z + a)
    Y = bf16(oracle.layer_norm(Z, blk.ln2_w, blk.ln2_b, hp.ln_eps))
    U = bf16(oracle.gelu_erf(oracle.linear(Y, blk.up_w, blk.up_b)))
    f = oracle.linear(U, blk.down_w, blk.down_b)
    if blk.ls2 is not None:
        f = f * blk.ls2
    return fp32(Z + f)


def encoder_forward_recipe(hp, w, pixels, n_layers=None):
    """The encoder forward with the recipe's roundings (tokens [B, N, D])."""
    px = np.asarray(pixels, dtype=np.float64)
    hi = bf16(px)
    px_split = hi + bf16(px - hi)
    rope_pos, visible = oracle.rope_and_mask(hp, pixels.shape)
    Z = fp32(oracle.embed(hp, w, px_split))
    L = len(w.blocks) if n_layers is None else n_layers
    for blk in w.blocks[:L]:
        Z = _block(Z, blk, hp, rope_pos, visible)
    return oracle.layer_norm(Z, w.norm_w, w.norm_b, hp.ln_eps)

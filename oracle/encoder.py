"""CPU oracle of the shared pre-LN ViT encoder forward, in numpy float64.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The library's own
compute path never calls it and shares no code with it.

Each function is the plain definition of one step of the encoder graph of
jepa.cpp "Architecture", section "The shared ViT graph":

    tokens = patch_embed(rearranged pixels) [+ pos] [+ cls] [+ modality vector]
    per block:  x += attn(ln1(x));  x += ffn(ln2(x))
    x = norm(x)

written out directly, with no blocking, fusion or reordering beyond what the
definition states.  Library primitives used as steps: numpy matmul (dgemm),
numpy exp/sin/cos, scipy's erf.  Attention is a dense masked softmax; it is
split over query rows only to bound memory (each row is independent).

Inputs are the exact values the GPU sees (bf16 weights arrive already rounded
and held in fp32); everything is promoted to float64 here.

Readings of points the pages leave open are listed next to the function
they affect ("Reading: ...").
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

# enumerations shared with the hyperparameter struct (values, not code)
POS_NONE, POS_TABLE = 0, 1
LAYOUT_TILED, LAYOUT_INTERLEAVED = 0, 1
ATTN_FULL, ATTN_BLOCK_CAUSAL = 0, 1


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# a1  patchify: rearrange NCTHW pixels into [B, Np, C*t*P*P]
#     jepa.cpp "Architecture", "The shared ViT graph" (rearrange + one matmul
#     equals the strided convolution); "GGUF schema (v1)", "Encoder tensors"
#     (C-T-H-W flattening); "GGUF schema (v1)", "Token order" (T, then H, then W)
# ---------------------------------------------------------------------------
def patchify(pixels: np.ndarray, tubelet: int, patch: int) -> np.ndarray:
    """A[b, n, f] = X[b, c, t'*t + dt, h'*P + dh, w'*P + dw] with
    n = (t'*gh + h')*gw + w' and f = ((c*t + dt)*P + dh)*P + dw."""
    B, C, T, H, W = pixels.shape
    gt, gh, gw = T // tubelet, H // patch, W // patch
    assert gt * tubelet == T and gh * patch == H and gw * patch == W
    x = pixels.reshape(B, C, gt, tubelet, gh, patch, gw, patch)
    # axes now: b, c, t', dt, h', dh, w', dw  ->  b, t', h', w', c, dt, dh, dw
    x = x.transpose(0, 2, 4, 6, 1, 3, 5, 7)
    return x.reshape(B, gt * gh * gw, C * tubelet * patch * patch)


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x W^T + b for a PyTorch-row-major weight W [out, in]."""
    y = np.matmul(_f64(x), _f64(w).T)
    if b is not None:
        y = y + _f64(b)
    return y


# ---------------------------------------------------------------------------
# a4  LayerNorm, "GGUF schema (v1)" jepa.enc.ln_eps (1e-6);
#     "Architecture", "Attention and precision": the CPU reference uses a
#     centred two-pass variance.
#     Reading: population variance (divide by D), eps inside the square root.
# ---------------------------------------------------------------------------
def layer_norm(x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * _f64(w) + _f64(b)


# ---------------------------------------------------------------------------
# a9  GELU, exact erf form ("GGUF schema (v1)", jepa.enc.act = gelu_erf)
# ---------------------------------------------------------------------------
def gelu_erf(x: np.ndarray) -> np.ndarray:
    x = _f64(x)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


# ---------------------------------------------------------------------------
# a6  3-D RoPE, jepa.cpp "Architecture", section "3-D RoPE"; schema keys
#     rope_freq_layout / rope_interpolate / rope_ref_grid; SkyVision.cpp
#     README, section "V-JEPA 2" (segment order t, h, w, then the untouched
#     dims; the odd-length wrap of the tiled table).
# ---------------------------------------------------------------------------
def rope_rotated_dims(head_dim: int) -> int:
    """Rotated dims per axis: d = 2*((head_dim // 3) // 2)."""
    return 2 * ((head_dim // 3) // 2)


def rope_frequencies(d: int, theta: float = 10000.0) -> np.ndarray:
    """omega_k = 1 / theta**(2k/d), k in [0, d/2)."""
    k = np.arange(d // 2, dtype=np.float64)
    return 1.0 / theta ** (2.0 * k / d)


def rope_freq_index(d: int, layout: int) -> np.ndarray:
    """Frequency index used by element j of an axis segment of length d.
    tiled:       table[j] = f(pos * omega_{j mod d/2})
    interleaved: table[2k] = table[2k+1] = f(pos * omega_k)"""
    j = np.arange(d)
    if layout == LAYOUT_TILED:
        return j % (d // 2)
    if layout == LAYOUT_INTERLEAVED:
        return j // 2
    raise ValueError(layout)


def token_grid_positions(n_patches: int, grid: Sequence[int]):
    """Patch token i -> (t, h, w) with i = t*gh*gw + h*gw + w ("GGUF schema
    (v1)", "Token order"; "Architecture", "3-D RoPE").
    Reading: t is the tubelet-grid index, not the frame index."""
    gt, gh, gw = grid
    i = np.arange(n_patches)
    t = i // (gh * gw)
    h = (i % (gh * gw)) // gw
    w = i % gw
    return t.astype(np.float64), h.astype(np.float64), w.astype(np.float64)


def rope_interpolate_scale(ref_grid: int, g: int) -> float:
    """Scale applied to the h and w positions under interpolate_rope:
    (ref_grid - 1) / (g - 1).  Reading: a one-position axis (g = 1) keeps
    scale 1 (its only position is 0, the page's formula is 0/0 there)."""
    if g <= 1:
        return 1.0
    return (ref_grid - 1) / (g - 1)


def rope_positions(n_patches: int, grid: Sequence[int], interpolate: bool, ref_grid: int):
    t, h, w = token_grid_positions(n_patches, grid)
    if interpolate:
        _, gh, gw = grid
        h = h * rope_interpolate_scale(ref_grid, gh)
        w = w * rope_interpolate_scale(ref_grid, gw)
    return t, h, w


def rope_angles(pos: np.ndarray, d: int, layout: int, theta: float) -> np.ndarray:
    """[n, d] angles pos * omega_{k(j)} of one axis segment."""
    omega = rope_frequencies(d, theta)
    return np.outer(_f64(pos), omega[rope_freq_index(d, layout)])


def rotate90(seg: np.ndarray) -> np.ndarray:
    """rotate90 on interleaved pairs: (y1, y2) -> (-y2, y1)."""
    r = np.empty_like(seg)
    r[..., 0::2] = -seg[..., 1::2]
    r[..., 1::2] = seg[..., 0::2]
    return r


def rope3d_apply(x: np.ndarray, pos_thw, layout: int, theta: float) -> np.ndarray:
    """Rotate the patch rows of x [..., n, head_dim]: axis a in (t, h, w)
    occupies dims [a*d, (a+1)*d); out = x*cos + rotate90(x)*sin there; dims
    at and beyond 3*d pass through unchanged."""
    x = _f64(x)
    hd = x.shape[-1]
    d = rope_rotated_dims(hd)
    out = x.copy()
    for a, pos in enumerate(pos_thw):
        ang = rope_angles(pos, d, layout, theta)
        seg = x[..., a * d:(a + 1) * d]
        out[..., a * d:(a + 1) * d] = seg * np.cos(ang) + rotate90(seg) * np.sin(ang)
    return out


# ---------------------------------------------------------------------------
# a7  attention and the block-causal mask
#     "Architecture", "Block-causal attention"; "GGUF schema (v1)",
#     jepa.enc.attn_mode and the levjepa family note.
# ---------------------------------------------------------------------------
def frame_ids(n_tokens: int, n_prefix: int, tokens_per_frame: int) -> np.ndarray:
    """frame_id of each token: (id - prefix) // (gh*gw); -1 for prefix tokens."""
    i = np.arange(n_tokens)
    f = (i - n_prefix) // tokens_per_frame
    f[:n_prefix] = -1
    return f


def block_causal_visible(n_tokens: int, n_prefix: int, tokens_per_frame: int) -> np.ndarray:
    """visible[i, j]: the prefix (CLS) rows see every key; a patch query sees
    a patch key iff frame(query) >= frame(key); no patch query sees a prefix
    key (the CLS column is closed)."""
    f = frame_ids(n_tokens, n_prefix, tokens_per_frame)
    is_prefix = np.arange(n_tokens) < n_prefix
    vis = (f[:, None] >= f[None, :]) & ~is_prefix[None, :]
    vis |= is_prefix[:, None]
    return vis


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              visible: Optional[np.ndarray] = None, row_chunk: int = 2048) -> np.ndarray:
    """softmax(q k^T / sqrt(hd) [masked]) v for one head: q, k, v [N, hd].
    Reading: scale 1/sqrt(head_dim) ("Architecture": RoPE comes before the
    scaling).  A row with no visible key cannot occur for the masks defined
    here (every query sees at least its own frame); it is asserted."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    out = np.empty((N, v.shape[1]), dtype=np.float64)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        s = np.matmul(q[r0:r1], k.T) * scale
        if visible is not None:
            vis = visible[r0:r1]
            assert vis.any(axis=1).all(), "a query row with no visible key"
            s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[r0:r1] = np.matmul(p, v)
    return out


# ---------------------------------------------------------------------------
# the whole encoder
# ---------------------------------------------------------------------------
def _hp(hp, key, default=None):
    if isinstance(hp, dict):
        return hp.get(key, default)
    return getattr(hp, key, default)


def cubic_weights(t: float, a: float = -0.75):
    """Cubic-convolution weights of the four taps at offsets -1, 0, 1, 2 from
    floor(x), t = x - floor(x) (Keys' kernel with a = -0.75):
      W(s) = (a+2)|s|^3 - (a+3)|s|^2 + 1        for |s| <= 1
      W(s) = a|s|^3 - 5a|s|^2 + 8a|s| - 4a       for 1 < |s| < 2."""
    def W(s):
        s = abs(s)
        if s <= 1.0:
            return (a + 2.0) * s ** 3 - (a + 3.0) * s ** 2 + 1.0
        if s < 2.0:
            return a * s ** 3 - 5.0 * a * s ** 2 + 8.0 * a * s - 4.0 * a
        return 0.0
    return [W(1.0 + t), W(t), W(1.0 - t), W(2.0 - t)]


def resample_axis(x: np.ndarray, axis: int, n_out: int, mode: str) -> np.ndarray:
    """Resample one axis of x to n_out samples, sample centres aligned
    (align_corners off): output o reads source coordinate
    c = (o + 1/2) * n_in / n_out - 1/2.  'cubic': the four taps around c with
    cubic_weights, indices clamped to the axis; 'linear': the two taps around
    max(c, 0), the upper one clamped to the axis."""
    n_in = x.shape[axis]
    x = np.moveaxis(_f64(x), axis, 0)
    out = np.zeros((n_out,) + x.shape[1:])
    for o in range(n_out):
        c = (o + 0.5) * n_in / n_out - 0.5
        if mode == "cubic":
            i = math.floor(c)
            for k, wk in enumerate(cubic_weights(c - i)):
                out[o] += wk * x[min(max(i - 1 + k, 0), n_in - 1)]
        else:
            c = max(c, 0.0)
            i = math.floor(c)
            lam = c - i
            out[o] = (1.0 - lam) * x[min(i, n_in - 1)] + lam * x[min(i + 1, n_in - 1)]
    return np.moveaxis(out, 0, axis)


def interpolate_pos_table(pos: np.ndarray, n_prefix: int, src_grid, dst_grid, mode: int) -> np.ndarray:
    """A position table built for src_grid = (t, h, w), resampled to dst_grid
    (jepa.cpp "GGUF schema (v1)", "Encoder tensors": the runtime bicubic /
    trilinear-interpolates the precomputed table for other grids).  The
    prefix (CLS) rows are kept.  mode 1: bicubic over (h, w) of a one-frame
    table; mode 2: trilinear over (t, h, w).  Reading: sample centres aligned
    (align_corners off), cubic a = -0.75, the separable products of the axis
    resamplings."""
    pos = _f64(pos)
    D = pos.shape[1]
    t0, h0, w0 = src_grid
    t1, h1, w1 = dst_grid
    g = pos[n_prefix:n_prefix + t0 * h0 * w0].reshape(t0, h0, w0, D)
    if mode == 1:
        assert t0 == 1 and t1 == 1, "bicubic resampling of a one-frame table"
        g = resample_axis(resample_axis(g, 1, h1, "cubic"), 2, w1, "cubic")
    elif mode == 2:
        g = resample_axis(resample_axis(resample_axis(g, 0, t1, "linear"), 1, h1, "linear"), 2, w1, "linear")
    else:
        raise ValueError("unknown interpolation mode")
    return np.concatenate([pos[:n_prefix], g.reshape(t1 * h1 * w1, D)], axis=0)


def assemble_tokens(E: np.ndarray, hp, cls, pos, mod) -> np.ndarray:
    """a3: Z = [cls?; E] (+ pos) (+ mod).  The pos table rows are [CLS?;
    patches] ("GGUF schema (v1)", enc.pos_embed); a CLS with no table gets
    nothing.  Reading: the modality vector is added to every token after the
    position add ("Architecture", graph order)."""
    B, Np, D = E.shape
    p = 1 if _hp(hp, "cls_token") else 0
    Z = np.zeros((B, Np + p, D), dtype=np.float64)
    Z[:, p:] = E
    if p:
        Z[:, 0] = _f64(cls)
    if _hp(hp, "pos_type") == POS_TABLE:
        Z = Z + _f64(pos)[None, : Np + p]
    if _hp(hp, "modality_embed"):
        Z = Z + _f64(mod)[None, None, :]
    return Z


def encoder_block(Z: np.ndarray, blk, hp, rope_pos, visible) -> np.ndarray:
    """One pre-LN block: x += ls1*attn(ln1(x)); x += ls2*ffn(ln2(x))."""
    B, N, D = Z.shape
    H = _hp(hp, "n_head")
    hd = D // H
    eps = _hp(hp, "ln_eps")
    p = 1 if _hp(hp, "cls_token") else 0
    Y = layer_norm(Z, blk.ln1_w, blk.ln1_b, eps)
    qkv = linear(Y, blk.qkv_w, blk.qkv_b)                # [B, N, 3D], rows [q; k; v]
    q = qkv[..., 0:D].reshape(B, N, H, hd).transpose(0, 2, 1, 3)
    k = qkv[..., D:2 * D].reshape(B, N, H, hd).transpose(0, 2, 1, 3)
    v = qkv[..., 2 * D:3 * D].reshape(B, N, H, hd).transpose(0, 2, 1, 3)
    if rope_pos is not None:
        layout, theta = _hp(hp, "rope_layout"), _hp(hp, "rope_theta")
        q = q.copy(); k = k.copy()
        q[:, :, p:] = rope3d_apply(q[:, :, p:], rope_pos, layout, theta)
        k[:, :, p:] = rope3d_apply(k[:, :, p:], rope_pos, layout, theta)
    O = np.empty((B, H, N, hd))
    for b in range(B):
        for h in range(H):
            O[b, h] = attention(q[b, h], k[b, h], v[b, h], visible)
    O = O.transpose(0, 2, 1, 3).reshape(B, N, D)
    a = linear(O, blk.out_w, blk.out_b)
    if blk.ls1 is not None:
        a = a * _f64(blk.ls1)
    Z = Z + a
    Y = layer_norm(Z, blk.ln2_w, blk.ln2_b, eps)
    f = linear(gelu_erf(linear(Y, blk.up_w, blk.up_b)), blk.down_w, blk.down_b)
    if blk.ls2 is not None:
        f = f * _f64(blk.ls2)
    return Z + f


def is_image_input(hp, pixels_shape) -> bool:
    """An image (one frame) goes through the separate one-frame tokenizer
    when the model has one (jepa.cpp "GGUF schema (v1)", V-JEPA 2.1: a
    2x16x16 tubelet tokenizer and a 1x16x16 image tokenizer, with a modality
    vector per input kind).  Reading: the input kind is decided by the frame
    count, one frame being an image."""
    return bool(_hp(hp, "image_patch_embed", 0)) and pixels_shape[2] == 1


def geometry(hp, pixels_shape):
    B, C, T, H, W = pixels_shape
    P, t = _hp(hp, "patch_size"), _hp(hp, "tubelet_size")
    if is_image_input(hp, pixels_shape):
        t = 1
    grid = (T // t, H // P, W // P)
    n_patches = grid[0] * grid[1] * grid[2]
    p = 1 if _hp(hp, "cls_token") else 0
    return grid, n_patches, p


def rope_and_mask(hp, pixels_shape):
    grid, n_patches, p = geometry(hp, pixels_shape)
    rope_pos = None
    if _hp(hp, "rope"):
        rope_pos = rope_positions(n_patches, grid, bool(_hp(hp, "rope_interpolate")),
                                  _hp(hp, "rope_ref_grid"))
    visible = None
    if _hp(hp, "attn_mode") == ATTN_BLOCK_CAUSAL:
        visible = block_causal_visible(n_patches + p, p, grid[1] * grid[2])
    return rope_pos, visible


def position_table(hp, w, pixels_shape):
    """The table the tokens get: the stored one, or its resampling to the
    input grid when the model interpolates and the grids differ."""
    if _hp(hp, "pos_type") != POS_TABLE or not _hp(hp, "pos_interp", 0):
        return w.pos
    grid, _, p = geometry(hp, pixels_shape)
    src = (_hp(hp, "pos_grid_t"), _hp(hp, "pos_grid_h"), _hp(hp, "pos_grid_w"))
    if tuple(src) == tuple(grid):
        return w.pos
    return interpolate_pos_table(w.pos, p, src, grid, _hp(hp, "pos_interp"))


def embed(hp, w, pixels) -> np.ndarray:
    """a1-a3: patchify, patch GEMM with bias, token assembly (through the
    image tokenizer and with the image modality vector for an image input of
    a model that has them)."""
    if is_image_input(hp, pixels.shape):
        A = patchify(_f64(pixels), 1, _hp(hp, "patch_size"))
        E = linear(A, w.patch_img_w, w.patch_img_b)
        return assemble_tokens(E, hp, w.cls, position_table(hp, w, pixels.shape), w.mod_img)
    A = patchify(_f64(pixels), _hp(hp, "tubelet_size"), _hp(hp, "patch_size"))
    E = linear(A, w.patch_w, w.patch_b)
    return assemble_tokens(E, hp, w.cls, position_table(hp, w, pixels.shape), w.mod)


def pool(out: np.ndarray, hp) -> np.ndarray:
    """a11 pooled feature: the CLS row when the model has one, else the mean
    of the patch tokens ("GGUF schema (v1)" family notes ijepa / hfvit /
    levjepa; SkyVision.cpp README "V-JEPA 2": mean-pooled features)."""
    if _hp(hp, "cls_token"):
        return out[:, 0].copy()
    return out.mean(axis=1)


def encoder_forward(hp, w, pixels, n_layers: Optional[int] = None, return_residual=False, return_hier=False):
    """Full forward: returns (tokens [B, N, D], pooled [B, D]) in float64;
    with return_hier also the hierarchical outputs [n_hier, B, N, D]: the
    output of block hier_layers[k] through its own norm k ("GGUF schema
    (v1)", enc.hier_norm.{k}: one norm per hierarchical layer; V-JEPA 2.1)."""
    rope_pos, visible = rope_and_mask(hp, pixels.shape)
    Z = embed(hp, w, pixels)
    L = len(w.blocks) if n_layers is None else n_layers
    hier_layers = list(_hp(hp, "hier_layers", ()) or ())
    hier = []
    for l, blk in enumerate(w.blocks[:L]):
        Z = encoder_block(Z, blk, hp, rope_pos, visible)
        if l in hier_layers:
            k = hier_layers.index(l)
            hier.append(layer_norm(Z, w.hier_norm_w[k], w.hier_norm_b[k], _hp(hp, "ln_eps")))
    out = layer_norm(Z, w.norm_w, w.norm_b, _hp(hp, "ln_eps"))
    res = (out, pool(out, hp))
    if return_residual:
        res = res + (Z,)
    if return_hier:
        res = res + (np.stack(hier) if hier else np.zeros((0,) + out.shape),)
    return res


def encoder_block_rows(Z: np.ndarray, blk, hp, rope_pos, visible, rows: np.ndarray) -> np.ndarray:
    """The block's output on selected token rows only (every row's output
    depends on all rows' keys and values, which are computed in full; the
    queries, the output projection and the FFN are evaluated on `rows` only).
    Used to check a full-size layer one sampled token at a time."""
    B, N, D = Z.shape
    H = _hp(hp, "n_head")
    hd = D // H
    eps = _hp(hp, "ln_eps")
    p = 1 if _hp(hp, "cls_token") else 0
    Wq, Wk, Wv = blk.qkv_w[0:D], blk.qkv_w[D:2 * D], blk.qkv_w[2 * D:3 * D]
    bq, bk, bv = blk.qkv_b[0:D], blk.qkv_b[D:2 * D], blk.qkv_b[2 * D:3 * D]
    Y = layer_norm(Z, blk.ln1_w, blk.ln1_b, eps)
    k = linear(Y, Wk, bk).reshape(B, N, H, hd).transpose(0, 2, 1, 3)
    v = linear(Y, Wv, bv).reshape(B, N, H, hd).transpose(0, 2, 1, 3)
    q = linear(Y[:, rows], Wq, bq).reshape(B, len(rows), H, hd).transpose(0, 2, 1, 3)
    if rope_pos is not None:
        layout, theta = _hp(hp, "rope_layout"), _hp(hp, "rope_theta")
        k = k.copy()
        k[:, :, p:] = rope3d_apply(k[:, :, p:], rope_pos, layout, theta)
        patch_rows = rows >= p
        if patch_rows.any():
            sel = [pp[rows[patch_rows] - p] for pp in rope_pos]
            q[:, :, patch_rows] = rope3d_apply(q[:, :, patch_rows], sel, layout, theta)
    vis = None if visible is None else visible[rows]
    O = np.empty((B, H, len(rows), hd))
    for b in range(B):
        for h in range(H):
            O[b, h] = attention(q[b, h], k[b, h], v[b, h], vis)
    O = O.transpose(0, 2, 1, 3).reshape(B, len(rows), D)
    a = linear(O, blk.out_w, blk.out_b)
    if blk.ls1 is not None:
        a = a * _f64(blk.ls1)
    Zr = _f64(Z[:, rows]) + a
    Yr = layer_norm(Zr, blk.ln2_w, blk.ln2_b, eps)
    f = linear(gelu_erf(linear(Yr, blk.up_w, blk.up_b)), blk.down_w, blk.down_b)
    if blk.ls2 is not None:
        f = f * _f64(blk.ls2)
    return Zr + f


def compare(gpu: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    """Gate statistics between a result and the oracle over the last axis:
    rel = max|g - o| / max|o|, maxabs = max|g - o|, and the minimum per-token
    cosine."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, gpu.shape[-1])
    o = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    diff = np.abs(g - o)
    maxabs = float(diff.max()) if diff.size else 0.0
    rel = maxabs / max(float(np.abs(o).max()), 1e-300) if diff.size else 0.0
    num = (g * o).sum(axis=1)
    den = np.sqrt((g * g).sum(axis=1) * (o * o).sum(axis=1))
    cos = num / np.maximum(den, 1e-300)
    return {"rel": rel, "maxabs": maxabs, "min_cos": float(cos.min()) if cos.size else 1.0,
            "finite": bool(np.isfinite(g).all())}

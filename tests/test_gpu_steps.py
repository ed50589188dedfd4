"""Each step of the encoder on the GPU, called through its C-ABI entry point,
against the CPU oracle's definition of that step, on seeded inputs whose
sizes span several tiles and end in a ragged tail."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

from gpu_util import say, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(x, dtype=W.DTYPE_F32):
    from vision_transformer_amd.vitenc import to_device
    store, _ = W.quantise(np.asarray(x, np.float32), dtype)
    return to_device(store, dtype)


def exact(x, dtype):
    """The values a tensor of this dtype holds (what the GPU sees)."""
    return W.quantise(np.asarray(x, np.float32), dtype)[1].astype(np.float64)


def rel_err(g, o):
    return float(np.abs(g - o).max() / max(np.abs(o).max(), 1e-30))


# output-rounding bound of a stored 16-bit result plus fp32 accumulation noise
def out_tol(dtype):
    return {W.DTYPE_F32: 2e-6, W.DTYPE_BF16: 2 ** -8, W.DTYPE_F16: 2 ** -11}[dtype]


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16])
@pytest.mark.parametrize("M,D", [(37, 192), (130, 1024), (9, 1408), (5, 100), (7, 98), (3, 4096)])
def test_layernorm(gpu_lib, dtype, M, D):
    from vision_transformer_amd import vitenc as V
    say(f"layernorm dtype={dtype} M={M} D={D}")
    rng = np.random.default_rng(M * D)
    x = rng.standard_normal((M, D)).astype(np.float32) * 3 + 0.7
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D)).astype(np.float32)
    y = V.op_layernorm(dev(x), dev(w), dev(b), 1e-6, dtype)
    torch.cuda.synchronize()
    ref = oracle.layer_norm(x, w, b, 1e-6)
    g = to_np(y)
    assert np.abs(g - ref).max() <= out_tol(dtype) * np.abs(ref).max() + 1e-5


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16, W.DTYPE_F16])
@pytest.mark.parametrize("M,N,K", [(200, 192, 96), (257, 576, 192), (131, 320, 1024), (64, 130, 588)])
def test_linear_gelu_and_residual(gpu_lib, dtype, M, N, K):
    from vision_transformer_amd import vitenc as V
    say(f"linear dtype={dtype} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    Wt = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    ls = (1 + 0.2 * rng.standard_normal(N)).astype(np.float32)
    Ae, We = exact(A, dtype), exact(Wt, dtype)
    U = V.op_linear_gelu(dtype, dev(A, dtype), dev(Wt, dtype), dev(b))
    Z0 = rng.standard_normal((M, N)).astype(np.float32)
    Zd = dev(Z0)
    V.op_linear_residual(dtype, dev(A, dtype), dev(Wt, dtype), dev(b), Zd, ls=dev(ls))
    Z2 = dev(Z0)
    V.op_linear_residual(dtype, dev(A, dtype), dev(Wt, dtype), dev(b), Z2)
    torch.cuda.synchronize()
    lin = oracle.linear(Ae, We, b)
    ref_u = oracle.gelu_erf(lin)
    scale = np.abs(lin).max()
    acc_tol = 1e-5 * scale
    assert np.abs(to_np(U) - ref_u).max() <= out_tol(dtype) * np.abs(ref_u).max() + acc_tol
    assert np.abs(to_np(Zd) - (Z0 + ls * lin)).max() <= acc_tol * 4 + 1e-6
    assert np.abs(to_np(Z2) - (Z0 + lin)).max() <= acc_tol * 4 + 1e-6


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16])
@pytest.mark.parametrize("geo", [
    dict(B=2, T=4, H=48, Wd=32, tub=2, P=16, cls=False, pos=False, mod=True),
    dict(B=1, T=1, H=56, Wd=42, tub=1, P=14, cls=True, pos=True, mod=False),
    dict(B=3, T=2, H=32, Wd=32, tub=1, P=16, cls=True, pos=False, mod=True),
    dict(B=2, T=2, H=24, Wd=40, tub=2, P=8, cls=False, pos=True, mod=False),
])
def test_embed(gpu_lib, dtype, geo):
    from vision_transformer_amd import vitenc as V
    say(f"embed dtype={dtype} {geo}")
    rng = np.random.default_rng(5)
    B, T, H, Wd, tub, P = geo["B"], geo["T"], geo["H"], geo["Wd"], geo["tub"], geo["P"]
    C, D = 3, 192
    px = rng.standard_normal((B, C, T, H, Wd)).astype(np.float32)
    K = C * tub * P * P
    pw = (rng.standard_normal((D, K)) * 0.02).astype(np.float32)
    pb = (rng.standard_normal(D) * 0.02).astype(np.float32)
    Np = (T // tub) * (H // P) * (Wd // P)
    p = 1 if geo["cls"] else 0
    pos = rng.standard_normal((Np + p, D)).astype(np.float32) if geo["pos"] else None
    cls = rng.standard_normal(D).astype(np.float32) if geo["cls"] else None
    mod = rng.standard_normal(D).astype(np.float32) if geo["mod"] else None
    Z = V.op_embed(dtype, dev(px), tub, P, dev(pw, dtype), dev(pb), pos=None if pos is None else dev(pos),
                   cls=None if cls is None else dev(cls), mod=None if mod is None else dev(mod))
    torch.cuda.synchronize()
    hp = dict(cls_token=p, pos_type=1 if pos is not None else 0, modality_embed=1 if mod is not None else 0,
              tubelet_size=tub, patch_size=P)
    # 16-bit embeddings with K a multiple of 64 carry each pixel as hi + lo
    # (about 16 significant bits): compare them with the fp32 pixels; otherwise
    # the pixels enter rounded to the model dtype
    split = dtype != W.DTYPE_F32 and K % 64 == 0
    E = oracle.linear(oracle.patchify(px if split else exact(px, dtype), tub, P), exact(pw, dtype), pb)
    ref = oracle.assemble_tokens(E, hp, cls, pos, mod)
    assert np.abs(to_np(Z) - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-6


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16])
@pytest.mark.parametrize("case", [
    dict(B=2, grid=(3, 2, 5), p=0, layout=W.LAYOUT_TILED, interp=0, hd=64, H=2),
    dict(B=1, grid=(2, 5, 3), p=1, layout=W.LAYOUT_TILED, interp=0, hd=64, H=3),
    dict(B=1, grid=(4, 6, 6), p=0, layout=W.LAYOUT_INTERLEAVED, interp=1, hd=64, H=2),
    dict(B=2, grid=(2, 3, 4), p=1, layout=W.LAYOUT_TILED, interp=0, hd=32, H=4),
    dict(B=1, grid=(1, 7, 9), p=0, layout=W.LAYOUT_INTERLEAVED, interp=0, hd=32, H=2),
    dict(B=2, grid=(2, 2, 2), p=1, layout=None, interp=0, hd=64, H=2),
])
def test_qkv_rope(gpu_lib, dtype, case):
    from vision_transformer_amd import vitenc as V
    say(f"qkv_rope dtype={dtype} {case}")
    rng = np.random.default_rng(7)
    B, (gt, gh, gw), p, hd, H = case["B"], case["grid"], case["p"], case["hd"], case["H"]
    D = H * hd
    N = gt * gh * gw + p
    Y = rng.standard_normal((B * N, D)).astype(np.float32)
    Wq = (rng.standard_normal((3 * D, D)) * 0.1).astype(np.float32)
    bq = (rng.standard_normal(3 * D) * 0.1).astype(np.float32)
    rope = case["layout"] is not None
    Q, K, Vt = V.op_qkv_rope(dtype, dev(Y, dtype), dev(Wq, dtype), dev(bq), B, N, H, rope=int(rope),
                             rope_layout=case["layout"] or 0, rope_interpolate=case["interp"], rope_ref_grid=4,
                             grid=(gt, gh, gw), n_prefix=p)
    torch.cuda.synchronize()
    qkv = oracle.linear(exact(Y, dtype), exact(Wq, dtype), bq).reshape(B, N, 3, H, hd)
    q = qkv[:, :, 0].transpose(0, 2, 1, 3)
    k = qkv[:, :, 1].transpose(0, 2, 1, 3)
    v = qkv[:, :, 2].transpose(0, 2, 1, 3)
    if rope:
        pos = oracle.rope_positions(gt * gh * gw, (gt, gh, gw), bool(case["interp"]), 4)
        q = q.copy(); k = k.copy()
        q[:, :, p:] = oracle.rope3d_apply(q[:, :, p:], pos, case["layout"], 1e4)
        k[:, :, p:] = oracle.rope3d_apply(k[:, :, p:], pos, case["layout"], 1e4)
    tol = out_tol(dtype) * 2
    for got, ref in ((to_np(Q), q), (to_np(K), k), (to_np(Vt)[..., :N].transpose(0, 1, 3, 2), v)):
        assert np.abs(got - ref).max() <= tol * np.abs(ref).max() + 1e-5


@pytest.mark.parametrize("dtype", [W.DTYPE_F32, W.DTYPE_BF16, W.DTYPE_F16])
@pytest.mark.parametrize("case", [
    dict(B=1, H=2, N=257, hd=64, mode=0, p=0, S=0),
    dict(B=2, H=1, N=64, hd=64, mode=0, p=0, S=0),
    dict(B=1, H=2, N=300, hd=32, mode=0, p=0, S=0),
    dict(B=1, H=2, N=1 + 5 * 40, hd=64, mode=1, p=1, S=40),
    dict(B=2, H=1, N=4 * 36, hd=64, mode=1, p=0, S=36),
    dict(B=1, H=1, N=1 + 3 * 100, hd=32, mode=1, p=1, S=100),
    dict(B=1, H=1, N=1 + 6 * 4, hd=64, mode=1, p=1, S=4),
    dict(B=1, H=2, N=257, hd=64, mode=0, p=1, S=0),
    dict(B=1, H=2, N=1 + 4 * 256, hd=64, mode=1, p=1, S=256),
    dict(B=2, H=1, N=1 + 33, hd=32, mode=0, p=1, S=0),
    # 16-bit calls split their late query tiles over two halves of the keys:
    # frames that straddle query tiles, a ragged last query tile and key tile
    dict(B=2, H=3, N=1 + 6 * 200, hd=64, mode=1, p=1, S=200),
    dict(B=1, H=2, N=8 * 128, hd=32, mode=1, p=0, S=128),
    # a split query tile whose earliest rows see no key in the second half of
    # its keys while later rows of the same wave do (frames of 300 tokens)
    dict(B=1, H=2, N=1 + 4 * 300, hd=64, mode=1, p=1, S=300),
    dict(B=1, H=2, N=1 + 4 * 300, hd=32, mode=1, p=1, S=300),
])
def test_attention(gpu_lib, dtype, case):
    _attention_case(dtype, case)


@pytest.mark.parametrize("dtype", [W.DTYPE_BF16, W.DTYPE_F16])
@pytest.mark.parametrize("case", [
    dict(B=1, H=2, N=1 + 16 * 256, hd=64, mode=1, p=1, S=256),
    dict(B=1, H=1, N=4096, hd=32, mode=0, p=0, S=0),
])
def test_attention_long_keys(gpu_lib, dtype, case):
    """From 4096 keys on, the 16-bit kernel issues its tile loads from
    inline assembly: a block-causal 4097-token clip with its CLS row (split
    halves, prefix runs) and a full-attention hd-32 case."""
    _attention_case(dtype, case)


@pytest.mark.parametrize("dtype", [W.DTYPE_BF16, W.DTYPE_F16])
@pytest.mark.parametrize("B,H,N,hd,p", [(1, 49, 2048, 64, 0), (1, 49, 2048, 32, 0), (1, 25, 4096, 64, 0),
                                          (1, 25, 4097, 64, 1), (2, 25, 2048, 64, 0)])
def test_attention_last_round_split(gpu_lib, dtype, B, H, N, hd, p):
    """Full attention whose grid of equal-cost query tiles exceeds the 768
    resident workgroups by a nearly empty last round (49 heads x 16 tiles =
    784, 25 x 32 = 800): the last tile or two of every head run as two
    halves over the keys and are merged.  Every row of the last two query
    tiles of each head and a sample of the other rows against the oracle;
    the 4096-key cases take the inline-assembly tile loads, the 4097-token
    one has a CLS row, whose runs of keys the same merge launch combines, and
    the two-item one (2 x 25 x 16 = 800 tiles) splits the last tile of every
    (item, head)."""
    from vision_transformer_amd import vitenc as V
    say(f"attention last-round split dtype={dtype} B={B} H={H} N={N} hd={hd} p={p}")
    rng = np.random.default_rng(N + H)
    q = rng.standard_normal((B, H, N, hd)).astype(np.float32)
    k = rng.standard_normal((B, H, N, hd)).astype(np.float32)
    v = rng.standard_normal((B, H, N, hd)).astype(np.float32)
    ldv = (N + 63) // 64 * 64
    vt = np.zeros((B, H, hd, ldv), np.float32)
    vt[..., :N] = v.transpose(0, 1, 3, 2)
    O = V.op_attention(dtype, dev(q, dtype), dev(k, dtype), dev(vt, dtype), attn_mode=0, n_prefix=p,
                       tokens_per_frame=0)
    torch.cuda.synchronize()
    g = to_np(O)
    qe, ke, ve = exact(q, dtype), exact(k, dtype), exact(v, dtype)
    rows = np.concatenate([np.arange(p), np.sort(p + rng.choice(N - 256 - p, 48, replace=False)),
                           np.arange(N - 256, N)])
    tol = {W.DTYPE_BF16: 1.5e-2, W.DTYPE_F16: 2e-3}[dtype]
    for b in range(B):
        for h in range(H):
            ref = oracle.attention(qe[b, h][rows], ke[b, h], ve[b, h])
            err = np.abs(g[b, rows, h * hd:(h + 1) * hd] - ref).max()
            assert err <= tol, (b, h, err)


def _attention_case(dtype, case):
    from vision_transformer_amd import vitenc as V
    say(f"attention dtype={dtype} {case}")
    rng = np.random.default_rng(case["N"])
    B, H, N, hd = case["B"], case["H"], case["N"], case["hd"]
    q = rng.standard_normal((B, H, N, hd)).astype(np.float32)
    k = rng.standard_normal((B, H, N, hd)).astype(np.float32)
    v = rng.standard_normal((B, H, N, hd)).astype(np.float32)
    ldv = (N + 63) // 64 * 64
    vt = np.zeros((B, H, hd, ldv), np.float32)
    vt[..., :N] = v.transpose(0, 1, 3, 2)
    O = V.op_attention(dtype, dev(q, dtype), dev(k, dtype), dev(vt, dtype), attn_mode=case["mode"],
                       n_prefix=case["p"], tokens_per_frame=case["S"])
    torch.cuda.synchronize()
    vis = oracle.block_causal_visible(N, case["p"], case["S"]) if case["mode"] == 1 else None
    qe, ke, ve = exact(q, dtype), exact(k, dtype), exact(v, dtype)
    ref = np.empty((B, N, H * hd))
    for b in range(B):
        for h in range(H):
            ref[b, :, h * hd:(h + 1) * hd] = oracle.attention(qe[b, h], ke[b, h], ve[b, h], vis)
    g = to_np(O)
    err = np.abs(g - ref).max()
    # P is rounded to the operand type before the PV product; the output is stored in it
    tol = {W.DTYPE_F32: 2e-5, W.DTYPE_BF16: 1.5e-2, W.DTYPE_F16: 2e-3}[dtype]
    assert err <= tol, err


@pytest.mark.parametrize("cls,p", [(1, 1), (0, 0), (0, 1)])
def test_pool(gpu_lib, cls, p):
    from vision_transformer_amd import vitenc as V
    rng = np.random.default_rng(3)
    X = rng.standard_normal((3, 77, 130)).astype(np.float32)
    got = to_np(V.op_pool(dev(X), cls, p))
    ref = X[:, 0] if cls else X[:, p:].astype(np.float64).mean(1)
    assert np.abs(got - ref).max() < 1e-5


@pytest.mark.parametrize("dtype", [W.DTYPE_BF16, W.DTYPE_F16])
@pytest.mark.parametrize("M,N,K", [(4133, 4096, 256), (4000, 3072, 256), (1990, 2048, 384), (2048, 2040, 320)])
def test_linear_wide_tiles(gpu_lib, dtype, M, N, K):
    """Shapes with enough tiles for the 256 x 256 direct-to-LDS kernel, with a
    ragged last row block (M = 4133); for 1.5 rounds of its 128 x 128 tiles
    (width 3072, the last row block ragged); and for one 128 x 128 tile per
    CU with its deeper slab ring, with ragged rows (M = 1990) or ragged
    columns (N = 2040)."""
    from vision_transformer_amd import vitenc as V
    say(f"linear wide dtype={dtype} M={M} N={N} K={K}")
    rng = np.random.default_rng(11)
    A = rng.standard_normal((M, K)).astype(np.float32)
    Wt = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    ls = (1 + 0.2 * rng.standard_normal(N)).astype(np.float32)
    Ae, We = exact(A, dtype), exact(Wt, dtype)
    U = V.op_linear_gelu(dtype, dev(A, dtype), dev(Wt, dtype), dev(b))
    Z0 = rng.standard_normal((M, N)).astype(np.float32)
    Zd = dev(Z0)
    V.op_linear_residual(dtype, dev(A, dtype), dev(Wt, dtype), dev(b), Zd, ls=dev(ls))
    torch.cuda.synchronize()
    lin = oracle.linear(Ae, We, b)
    ref_u = oracle.gelu_erf(lin)
    acc_tol = 1e-5 * np.abs(lin).max()
    assert np.abs(to_np(U) - ref_u).max() <= out_tol(dtype) * np.abs(ref_u).max() + acc_tol
    assert np.abs(to_np(Zd) - (Z0 + ls * lin)).max() <= acc_tol * 4 + 1e-6


def test_qkv_rope_wide_tiles(gpu_lib):
    """QKV at 2 x 2047 tokens (CLS + 2 x 31 x 33 grid), D 1024: the
    direct-to-LDS kernel at the ViT-L shape with the RoPE epilogue, a CLS row
    in each item and a ragged last row block."""
    from vision_transformer_amd import vitenc as V
    dtype = W.DTYPE_BF16
    B, (gt, gh, gw), p, H, hd = 2, (2, 31, 33), 1, 16, 64
    D = H * hd
    N = gt * gh * gw + p
    say(f"qkv_rope wide B={B} N={N} D={D}")
    rng = np.random.default_rng(13)
    Y = rng.standard_normal((B * N, D)).astype(np.float32)
    Wq = (rng.standard_normal((3 * D, D)) * 0.05).astype(np.float32)
    bq = (rng.standard_normal(3 * D) * 0.1).astype(np.float32)
    Q, K, Vt = V.op_qkv_rope(dtype, dev(Y, dtype), dev(Wq, dtype), dev(bq), B, N, H, rope=1,
                             rope_layout=W.LAYOUT_TILED, grid=(gt, gh, gw), n_prefix=p)
    torch.cuda.synchronize()
    qkv = oracle.linear(exact(Y, dtype), exact(Wq, dtype), bq).reshape(B, N, 3, H, hd)
    q = qkv[:, :, 0].transpose(0, 2, 1, 3).copy()
    k = qkv[:, :, 1].transpose(0, 2, 1, 3).copy()
    v = qkv[:, :, 2].transpose(0, 2, 1, 3)
    pos = oracle.rope_positions(gt * gh * gw, (gt, gh, gw), False, 0)
    q[:, :, p:] = oracle.rope3d_apply(q[:, :, p:], pos, W.LAYOUT_TILED, 1e4)
    k[:, :, p:] = oracle.rope3d_apply(k[:, :, p:], pos, W.LAYOUT_TILED, 1e4)
    tol = out_tol(dtype) * 2
    for got, ref in ((to_np(Q), q), (to_np(K), k), (to_np(Vt)[..., :N].transpose(0, 1, 3, 2), v)):
        assert np.abs(got - ref).max() <= tol * np.abs(ref).max() + 1e-5

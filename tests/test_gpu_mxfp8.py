"""8-bit block weights on the GPU, through the C ABI, against the oracle:
the quantiser bit for bit (every code and scale byte), the projections with
8-bit weights at shapes that select every GEMM tile configuration and end in
ragged tails, and the encoder forward with its four block matrices in 8 bits
(the oracle quantises the same fp32 draws with its own quantiser and runs
its forward on the dequantised values)."""
import numpy as np
import pytest

import oracle
from oracle import quant as Q
from vision_transformer_amd import workloads as W

from gpu_util import COS_BF16, ABS_BF16, say, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def gpu_quantize(w):
    from vision_transformer_amd import vitenc as V
    codes, scales = V.quantize_mxfp8(f32(w))
    torch.cuda.synchronize()
    R, C = w.shape
    s = scales.cpu().numpy().transpose(1, 0, 2).reshape(R, C // 32)   # -> [rows, blocks]
    return codes.cpu().numpy(), s


def _edge_matrix():
    vals = Q.e4m3_decode(np.arange(0, 0x7F))
    ties = (vals[1:-1] + vals[2:]) / 2
    w = np.concatenate([vals, ties, -vals, -ties])
    w = np.resize(w, (len(w) // 64 + 1) * 64).reshape(-1, 64)
    w[:, 0] = 448.0
    rng = np.random.default_rng(5)
    extra = np.zeros((8, 64))
    extra[0, :2] = [2.0 ** -127, -2.0 ** -128]    # clamped tiny block
    extra[1, 0] = 2.0 ** 127                      # clamped huge block: saturates
    extra[2, :] = -0.0
    extra[3, 5], extra[3, 6] = 448 * 2.0 ** -20, 449 * 2.0 ** -20
    extra[4, :] = 1e-39 * rng.standard_normal(64)   # fp32 subnormals
    return np.concatenate([w, w * 2.0 ** -20, w * 2.0 ** 10, extra])


@pytest.mark.parametrize("case", ["edges", "gauss_1024x4096", "gauss_4224x1408", "wide_range"])
def test_quantizer_bit_exact(gpu_lib, case):
    say(f"quantize {case}")
    rng = np.random.default_rng(hash(case) % 2 ** 32)
    w = {"edges": _edge_matrix,
         "gauss_1024x4096": lambda: rng.standard_normal((1024, 4096)) * 0.02,
         "gauss_4224x1408": lambda: rng.standard_normal((4224, 1408)) * 0.02,
         "wide_range": lambda: rng.standard_normal((96, 256)) * 2.0 ** rng.integers(-60, 60, (96, 256)),
         }[case]().astype(np.float32)
    codes, scales = gpu_quantize(w)
    c0, s0 = Q.mxfp8_quantize(w.astype(np.float64))
    assert np.array_equal(scales, s0), np.argwhere(scales != s0)[:5]
    bad = np.argwhere(codes != c0)
    assert len(bad) == 0, (bad[:5], codes[tuple(bad[:5].T)], c0[tuple(bad[:5].T)])


def _bf16_exact(x):
    return W.quantise(np.asarray(x, np.float32), W.DTYPE_BF16)


# M, N, K chosen for the tile each selects: 64 x 64 (few tiles), 128 x 128 with
# three stages (one tile per CU), 128 x 128, 256 x 256; ragged M and N tails
@pytest.mark.parametrize("M,N,K", [(196, 1024, 1024), (37, 1000, 1408), (2000, 1024, 4096), (1568, 4096, 1024),
                                   (4000, 4096, 1024), (1, 384, 384)])
def test_linear_8bit_weights(gpu_lib, M, N, K):
    from vision_transformer_amd import vitenc as V
    say(f"linear 8-bit M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N + K)
    A_store, A = _bf16_exact(rng.standard_normal((M, K)))
    Wt = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    ls = (1 + 0.2 * rng.standard_normal(N)).astype(np.float32)
    Ad = V.to_device(A_store, W.DTYPE_BF16)
    codes, scales = V.quantize_mxfp8(f32(Wt))
    U = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    V.op_linear_mxfp8(1, Ad, codes, scales, f32(b), U)
    Z0 = rng.standard_normal((M, N)).astype(np.float32)
    Zd = f32(Z0)
    V.op_linear_mxfp8(0, Ad, codes, scales, f32(b), Zd, ls=f32(ls))
    torch.cuda.synchronize()
    We = Q.dequantized_matrix(Wt)
    lin = oracle.linear(A.astype(np.float64), We, b)
    ref_u = oracle.gelu_erf(lin)
    acc_tol = 1e-5 * np.abs(lin).max()
    assert np.abs(to_np(U) - ref_u).max() <= 2 ** -8 * np.abs(ref_u).max() + acc_tol
    assert np.abs(to_np(Zd) - (Z0 + ls * lin)).max() <= acc_tol * 4 + 1e-6


def _cos_maxabs(g, o):
    g = g.reshape(-1, g.shape[-1])
    o = o.reshape(-1, o.shape[-1])
    cos = (g * o).sum(1) / (np.linalg.norm(g, axis=1) * np.linalg.norm(o, axis=1))
    return float(cos.min()), float(np.abs(g - o).max())


def _encode(wl, items=None):
    from vision_transformer_amd.vitenc import Encoder
    enc = Encoder.from_workload(wl)
    out, pooled = enc.encode(f32(wl.pixels))
    torch.cuda.synchronize()
    res = to_np(out), to_np(pooled)
    enc.close()
    return res


@pytest.mark.parametrize("name,kw", [
    ("ijepa_image_4layers", dict(idx=1, n_layer=4, batch=2)),
    ("levjepa_blockcausal_cls_2layers", dict(idx=4, n_layer=2, frames=4, height=64, width=96)),
    ("vjepa2_video_layerscale_2layers", dict(idx=2, n_layer=2, frames=4, height=64, width=64, layer_scale=1)),
])
def test_encoder_8bit_weights_vs_oracle(gpu_lib, name, kw):
    kw = dict(kw)
    cfg = W.CONFIGS[kw.pop("idx")].replace(weight_format=W.WEIGHTS_MXFP8, **kw)
    say(f"encoder 8-bit {name}: {cfg.batch} x {cfg.n_tokens} tokens, {cfg.n_layer} layers")
    wl = W.make_workload(cfg)
    out, pooled = _encode(wl)
    ref, ref_pool = _oracle(cfg, wl)
    cos, mx = _cos_maxabs(out, ref)
    say(f"  min cos {cos:.6f} max abs {mx:.3g}")
    assert np.isfinite(out).all() and cos >= COS_BF16 and mx <= ABS_BF16
    # the quantisation itself moves the output much more than the GPU/oracle difference
    ref_plain = _oracle(cfg, wl, dequantize=False)[0]
    cos_q, _ = _cos_maxabs(ref, ref_plain)
    assert cos_q < cos


def _oracle(cfg, wl, dequantize=True):
    w = Q.dequantized_weights(wl.weights) if dequantize else wl.weights
    return oracle.encoder_forward(cfg, w, wl.pixels)


def test_full_size_image_batch_8bit_weights(gpu_lib):
    """The ViT-L/16 image encoder at its full size (8 x 196 tokens, 24
    layers) with 8-bit block weights, in the launch configuration the
    benchmark times; items 0 and 7 at the sampled rows the oracle stored
    (tests/golden/make_oracle_samples.py)."""
    import os
    cfg = W.CONFIGS[1].replace(weight_format=W.WEIGHTS_MXFP8)
    gold = np.load(os.path.join(os.path.dirname(__file__), "golden", f"oracle_{cfg.name}_mxfp8.npz"))
    assert int(gold["n_layer"]) == cfg.n_layer and int(gold["seed"]) == cfg.seed
    say(f"encoder 8-bit full size: {cfg.batch} x {cfg.n_tokens} tokens, {cfg.n_layer} layers")
    wl = W.make_workload(cfg)
    out, pooled = _encode(wl)
    items, rows = gold["items"], gold["rows"]
    cos, mx = _cos_maxabs(out[items][:, rows], gold["tokens"])
    say(f"  min cos {cos:.6f} max abs {mx:.3g}")
    assert np.isfinite(out).all() and cos >= COS_BF16 and mx <= ABS_BF16
    assert np.abs(pooled[items] - gold["pooled"]).max() <= ABS_BF16

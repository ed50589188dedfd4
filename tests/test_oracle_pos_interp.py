"""Pins of the position-table resampling of the oracle (jepa.cpp "GGUF schema
(v1)", "Encoder tensors": tables are precomputed for the training grid and
bicubic / trilinear-interpolated for other grids) against torch's
interpolate in float64 (a library special case with the same sample
alignment), and closed forms."""
import numpy as np
import pytest

import oracle
from vision_transformer_amd import workloads as W

torch = pytest.importorskip("torch")
F = torch.nn.functional


def _table(rng, prefix, grid, D):
    t, h, w = grid
    return rng.standard_normal((prefix + t * h * w, D))


@pytest.mark.parametrize("src,dst", [((14, 14), (16, 16)), ((16, 16), (20, 24)), ((16, 16), (9, 5)),
                                     ((7, 11), (7, 11)), ((2, 3), (13, 1))])
def test_bicubic_matches_torch(src, dst):
    rng = np.random.default_rng(0)
    D = 6
    pos = _table(rng, 1, (1,) + src, D)
    out = oracle.interpolate_pos_table(pos, 1, (1,) + src, (1,) + dst, 1)
    g = torch.from_numpy(pos[1:].reshape(1, src[0], src[1], D)).permute(0, 3, 1, 2)
    ref = F.interpolate(g, size=dst, mode="bicubic", align_corners=False)
    ref = ref.permute(0, 2, 3, 1).reshape(dst[0] * dst[1], D).numpy()
    assert np.array_equal(out[0], pos[0])
    assert np.abs(out[1:] - ref).max() < 1e-12


@pytest.mark.parametrize("src,dst", [((8, 14, 14), (4, 16, 16)), ((2, 4, 4), (5, 3, 7)), ((3, 5, 6), (3, 5, 6))])
def test_trilinear_matches_torch(src, dst):
    rng = np.random.default_rng(1)
    D = 5
    pos = _table(rng, 0, src, D)
    out = oracle.interpolate_pos_table(pos, 0, src, dst, 2)
    g = torch.from_numpy(pos.reshape(1, *src, D)).permute(0, 4, 1, 2, 3)
    ref = F.interpolate(g, size=dst, mode="trilinear", align_corners=False)
    ref = ref.permute(0, 2, 3, 4, 1).reshape(-1, D).numpy()
    assert np.abs(out - ref).max() < 1e-12


def test_resampling_closed_forms():
    """Equal grids are the identity; both kernels keep constants (their
    weights sum to one); linear resampling keeps an affine ramp exactly at
    every output sample whose source coordinate lies inside the grid."""
    rng = np.random.default_rng(2)
    pos = _table(rng, 0, (1, 6, 7), 3)
    assert np.array_equal(oracle.interpolate_pos_table(pos, 0, (1, 6, 7), (1, 6, 7), 1), pos)
    assert np.array_equal(oracle.interpolate_pos_table(pos, 0, (1, 6, 7), (1, 6, 7), 2), pos)
    const = np.full((42, 3), 0.37)
    for mode in (1, 2):
        out = oracle.interpolate_pos_table(const, 0, (1, 6, 7), (1, 11, 4), mode)
        assert np.abs(out - 0.37).max() < 1e-15
    n_in, n_out = 6, 10
    ramp = 2.0 + 3.0 * np.arange(n_in, dtype=np.float64)
    x = oracle.resample_axis(ramp[:, None], 0, n_out, "linear")[:, 0]
    for o in range(n_out):
        c = (o + 0.5) * n_in / n_out - 0.5
        if 0.0 <= c <= n_in - 1:
            assert abs(x[o] - (2.0 + 3.0 * c)) < 1e-12
    assert sum(oracle.cubic_weights(0.3)) == pytest.approx(1.0, abs=1e-15)


def test_encoder_uses_the_resampled_table():
    """A learned 16x16 table with a CLS row, encoded at a 20x24 grid: the
    tokens before the first block carry the resampled table."""
    cfg = W.CONFIGS[0].replace(n_layer=0, height=280, width=336, pos_interp=W.POS_INTERP_BICUBIC,
                               pos_grid=(1, 16, 16), embed_dim=24, n_head=3, ffn_dim=32)
    wl = W.make_workload(cfg)
    assert wl.weights.pos.shape[0] == 257
    Z = oracle.embed(cfg, wl.weights, wl.pixels)
    A = oracle.patchify(wl.pixels.astype(np.float64), 1, 14)
    E = oracle.linear(A, wl.weights.patch_w, wl.weights.patch_b)
    tab = oracle.interpolate_pos_table(wl.weights.pos, 1, (1, 16, 16), (1, 20, 24), 1)
    assert np.abs(Z[0, 1:] - (E[0] + tab[1:])).max() < 1e-12
    assert np.abs(Z[0, 0] - (wl.weights.cls + tab[0])).max() < 1e-12

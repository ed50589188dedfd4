"""Pins of the 8-bit block weight oracle (oracle/quant.py) against things other
than itself: PyTorch's float8_e4m3fn type (decode of every code, and its
round-to-nearest-even cast in the range where it does not saturate to NaN), an
exhaustive nearest-value search over the E4M3 grid, closed forms of the block
scale, a round trip, and the rounding error bound."""
import numpy as np
import pytest
import torch

from oracle import quant as Q


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    got, ref = Q.e4m3_decode(codes), _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    # closed forms of the format: largest 448, smallest normal 2^-6, smallest subnormal 2^-9, one
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert got[0xFE] == -448.0 and np.signbit(got[0x80]) and got[0x80] == 0.0


def test_encode_matches_torch_cast_in_range():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest even; below 464
    (the midpoint to the next binade, where it turns to NaN) it is the same
    rounding the format defines."""
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.uniform(-463.9, 463.9, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
        (np.arange(-600, 600) / 2.0 ** 9),              # dense grid over the subnormals and their ties
        Q.e4m3_decode(np.arange(0, 0x7F)) * 1.0,        # every representable value exactly
        (Q.e4m3_decode(np.arange(1, 0x7E)) + Q.e4m3_decode(np.arange(2, 0x7F))) / 2,  # every tie
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = Q.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(got, ref)


def _brute_nearest(a):
    """Nearest non-negative E4M3 value to a >= 0 by exhaustive search over the
    126 finite magnitudes; ties go to the even mantissa."""
    codes = np.arange(0, 0x7F)
    vals = Q.e4m3_decode(codes)
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    if len(best) > 1:
        best = [c for c in best if (codes[c] & 1) == 0]
    return codes[best[0]]


def test_encode_matches_exhaustive_search_and_saturates():
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.uniform(0, 448, 300), rng.uniform(0, 2.0 ** -5, 300),
                           Q.e4m3_decode(np.arange(1, 0x7E)) * (1 + 2.0 ** -4)])
    for a in vals:
        assert Q.e4m3_encode(a) == _brute_nearest(a), a
        assert Q.e4m3_encode(-a) == (_brute_nearest(a) | 0x80), a
    # saturation: everything at or above 448 (the format has no larger finite value) -> 0x7E
    assert np.all(Q.e4m3_encode(np.array([448.0, 449.0, 480.0, 511.9, 1e6])) == 0x7E)
    assert np.all(Q.e4m3_encode(np.array([-450.0, -1e9])) == 0xFE)


def test_block_scale_closed_forms():
    # a block whose largest magnitude is exactly 2^k gets e = k - 8 and that weight the code of 256 (0x78)
    for k in (-20, -3, 0, 1, 7, 30):
        w = np.zeros((1, 32))
        w[0, 5] = -2.0 ** k
        w[0, 6] = 2.0 ** (k - 1)
        codes, s = Q.mxfp8_quantize(w)
        assert s[0, 0] == k - 8 + 127
        assert codes[0, 5] == (0x78 | 0x80) and codes[0, 6] == 0x70   # 256 and 128
    # largest magnitude 448 * 2^j: e = j and the code of 448; just above it: e = j + 1, 224.5 -> 224
    for j in (-9, 0, 4):
        w = np.zeros((1, 32))
        w[0, 0] = 448.0 * 2.0 ** j
        codes, s = Q.mxfp8_quantize(w)
        assert s[0, 0] == j + 127 and codes[0, 0] == 0x7E
        w[0, 0] = 449.0 * 2.0 ** j
        codes, s = Q.mxfp8_quantize(w)
        assert s[0, 0] == j + 1 + 127 and codes[0, 0] == 0x76
    # all-zero block
    codes, s = Q.mxfp8_quantize(np.zeros((2, 64)))
    assert np.all(codes == 0) and np.all(s == -117 + 127)
    # clamps: a tiny block keeps e = -117 (its weights round to zero), a huge one e = 117 and saturates
    w = np.zeros((2, 32))
    w[0, :2] = [2.0 ** -127, -2.0 ** -128]       # 2^-10 and 2^-11 at the scale: ties and below go to 0
    w[1, 0] = 2.0 ** 127
    codes, s = Q.mxfp8_quantize(w)
    assert list(s[:, 0]) == [10, 244] and codes[0, 0] == 0x00 and codes[0, 1] == 0x80 and codes[1, 0] == 0x7E
    # blocks are 32 consecutive weights of one row: a large weight only moves its own block's scale
    w = np.ones((2, 96))
    w[1, 40] = 1000.0
    _, s = Q.mxfp8_quantize(w)
    assert list(s[0]) == [119, 119, 119] and list(s[1]) == [119, 129, 119]


def test_round_trip_of_representable_blocks():
    """Weights that are already code * 2^e, with one element per block in the
    top binade [256, 448], quantise back to exactly those codes and scales."""
    rng = np.random.default_rng(2)
    N, K = 8, 128
    codes = rng.integers(0, 0x7F, (N, K)).astype(np.uint8)      # finite, non-negative
    codes |= (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    codes[:, ::32] = (0x78 + rng.integers(0, 7, (N, K // 32))).astype(np.uint8)  # 256 .. 416
    codes[(codes & 0x7F) == 0] = 0                               # -0 is not produced from a +0 weight
    e = rng.integers(-30, 10, (N, K // 32))
    scales = (e + 127).astype(np.uint8)
    w = Q.mxfp8_dequantize(codes, scales)
    c2, s2 = Q.mxfp8_quantize(w)
    assert np.array_equal(s2, scales) and np.array_equal(c2, codes)


def test_rounding_error_bound():
    """|w - deq(q(w))| is at most half the E4M3 spacing at w's binade, scaled
    by the block's 2^e, and no weight saturates: every block's largest weight
    lands in (224, 448] * 2^e."""
    rng = np.random.default_rng(3)
    w = rng.standard_normal((16, 256)) * 0.02
    codes, scales = Q.mxfp8_quantize(w)
    d = Q.mxfp8_dequantize(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1).astype(np.float64)
    a = np.abs(w) / np.exp2(e)
    assert a.max() <= 448
    top = a.reshape(16, 8, 32).max(axis=2)
    assert np.all((top > 224) & (top <= 448))
    _, ex = np.frexp(a)
    half = np.exp2(np.maximum(ex - 1, -6) - 4.0) * np.exp2(e)
    assert np.all(np.abs(w - d) <= half)
    # the relative error of a Gaussian matrix is that of a 3-bit mantissa
    rel = np.linalg.norm(w - d) / np.linalg.norm(w)
    assert 0.005 < rel < 0.04


def test_dequantized_weights_replace_only_the_block_matrices():
    from vision_transformer_amd import workloads as W
    cfg = W.CONFIGS[1].replace(n_layer=2, batch=1)
    w = W.make_workload(cfg).weights
    d = Q.dequantized_weights(w)
    assert d.patch_w is w.patch_w and d.norm_w is w.norm_w and len(d.blocks) == 2
    for b0, b1 in zip(w.blocks, d.blocks):
        for n in ("qkv_w", "out_w", "up_w", "down_w"):
            m0, m1 = getattr(b0, n), getattr(b1, n)
            assert m1.shape == m0.shape and not np.array_equal(m0, m1)
            assert np.array_equal(m1, Q.mxfp8_dequantize(*Q.mxfp8_quantize(m0)))
        assert b1.qkv_b is b0.qkv_b and b1.ln1_w is b0.ln1_w

"""CPU oracle of the 8-bit block weight format (numpy, exact arithmetic).

TEST INFRASTRUCTURE ONLY, like oracle/encoder.py: imported by the test suite
and the benchmark's CPU-baseline leg, never by the library.

What is quantised, and how it is used, follows jepa.cpp "GGUF schema (v1)",
section "Quantization rules": only the 2-D matrices of the attention (fused
qkv, out) and of the FFN (up, down) are stored in 8 bits; norms, biases,
layer scales, tables, tokens and the patch embedding stay as they are.  The
pages' 8-bit format (q8_0) stores each run of 32 consecutive weights of a row
with one shared scale; "Family notes" (the paragraph on the f32 tier of a GPU)
adds that the quantised files are the fastest GPU path.

Reading (the pages do not define the block's arithmetic beyond that): a block
is 32 consecutive weights along a row (the input dimension), its codes are
8-bit floats in the OCP E4M3 layout (sign, 4 exponent bits with bias 7, 3
mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; 0x7F/0xFF are
NaN and there is no infinity; the largest magnitude is 448), and its scale is
a power of two 2^e stored as the byte e + 127 (the OCP Microscaling "E8M0"
scale).  As q8_0 maps a block's largest weight to its largest code, e is the
smallest exponent with amax <= 448 * 2^e (amax: the block's largest
magnitude), so no weight saturates; every weight is divided by 2^e and
rounded to the nearest E4M3 value, ties to the even mantissa.  (The OCP rule
floor(log2 amax) - 8 would clip the largest weight of about a fifth of all
blocks by up to 12.5 %.)  The code's sign bit is always the weight's sign (so
a negative weight that rounds to zero is 0x80).  e is clamped to [-117, 117]
and an all-zero block takes e = -117: the smallest nonzero dequantised weight,
2^-9 * 2^-117, is then bf16's smallest normal number, and the largest, at
most 448 * 2^117, stays finite (a block above that saturates).

The dequantised weight is code * 2^e, which a bf16 (8-bit significand) holds
exactly; that is the value the oracle's forward multiplies with.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32          # weights per block, along a row
E4M3_MAX = 448.0
SCALE_MIN_EXP, SCALE_MAX_EXP = -117, 117


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values by the format's definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ef == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(ef.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(v) -> np.ndarray:
    """Real values (float64) -> E4M3 codes: round to nearest, ties to the even
    mantissa, saturating at 448; the sign bit copies the sign of v."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    neg = np.signbit(v)
    _, ex = np.frexp(a)                      # a = f * 2^ex with f in [0.5, 1)
    binade = np.maximum(ex - 1, -6)          # floor(log2 a), subnormals share binade -6
    spacing = np.exp2(binade.astype(np.float64) - 3.0)
    units = np.round(a / spacing)            # numpy rounds halves to even
    q = units * spacing                      # the rounded magnitude (may step up a binade)
    q = np.minimum(q, E4M3_MAX)
    # encode q exactly: subnormal when below 2^-6
    _, qx = np.frexp(q)
    qb = qx - 1
    sub = q < 2.0 ** -6
    ef = np.where(sub, 0, qb + 7)
    mant = np.where(sub, np.round(q / 2.0 ** -9), np.round((q / np.exp2(qb.astype(np.float64)) - 1.0) * 8.0))
    code = (ef.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(q == 0, 0, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def block_exponents(w: np.ndarray) -> np.ndarray:
    """Shared exponent e of every 32-weight block of the rows of w [N, K]: the
    smallest integer with amax <= 448 * 2^e, clamped to [-117, 117] (all-zero
    blocks: -117).  With amax = f * 2^E (f in [0.5, 1)) and 448 = 0.875 * 2^9
    that is E - 9 when f <= 0.875, else E - 8."""
    N, K = w.shape
    assert K % BLOCK == 0
    amax = np.abs(w.astype(np.float64)).reshape(N, K // BLOCK, BLOCK).max(axis=2)
    f, ex = np.frexp(amax)
    e = np.where(amax > 0, ex - 9 + (f > 0.875), SCALE_MIN_EXP)
    return np.clip(e, SCALE_MIN_EXP, SCALE_MAX_EXP).astype(np.int64)


def mxfp8_quantize(w: np.ndarray):
    """w [N, K] -> (codes uint8 [N, K], scale bytes uint8 [N, K/32] = e + 127)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    e = block_exponents(w)
    scaled = w.reshape(N, K // BLOCK, BLOCK) / np.exp2(e.astype(np.float64))[:, :, None]
    codes = e4m3_encode(scaled).reshape(N, K)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [N, K], scale bytes [N, K/32]) -> float64 weights code * 2^e."""
    N, K = codes.shape
    e = scales.astype(np.int64) - 127
    v = e4m3_decode(codes).reshape(N, K // BLOCK, BLOCK) * np.exp2(e.astype(np.float64))[:, :, None]
    return v.reshape(N, K)


def dequantized_matrix(w: np.ndarray) -> np.ndarray:
    """The weights the forward multiplies with when w is stored in this format."""
    return mxfp8_dequantize(*mxfp8_quantize(w))


def dequantized_weights(w, names=("qkv_w", "out_w", "up_w", "down_w")):
    """A copy of encoder weights w whose block matrices are replaced by the
    values the 8-bit format stores for them (the matrices jepa.cpp "GGUF
    schema (v1)", "Quantization rules" quantises); everything else is shared."""
    import copy
    out = copy.copy(w)
    out.blocks = []
    for blk in w.blocks:
        b = copy.copy(blk)
        for n in names:
            setattr(b, n, dequantized_matrix(getattr(blk, n)))
        out.blocks.append(b)
    return out

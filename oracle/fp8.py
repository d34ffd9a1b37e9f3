"""OCP FP8 E4M3 ("e4m3fn") encoding and per-tensor quantisation, in numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name FP8 attention on low-precision matrix units ([FA-legal],
FlashAttention-3 paragraph; [IO-aware], "Flash Attention 2 and 3") but give no
recipe.  The reading taken here: one scale per tensor, s = max(absmax, 2^-120)
/ 448 computed in float32, codes = RNE-with-saturation of the float32 quotient
x / s.  E4M3 itself is the OCP 8-bit format: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, subnormals below 2^-6 in steps of 2^-9, no
infinities, the all-ones pattern S.1111.111 is NaN, largest finite 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
SCALE_FLOOR = np.float32(2.0 ** -120)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code, as float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode_rne_sat(x) -> np.ndarray:
    """Round each float to the nearest E4M3 value, ties to even mantissa.

    Magnitudes above 448 saturate to 448 (code 0x7E with the sign); NaN maps
    to 0x7F.  Zero keeps its sign.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    code = np.zeros(a.shape, dtype=np.int64)
    small = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; a result of 8 is the smallest normal (code 8)
    code = np.where(small, np.rint(a / 2.0 ** -9).astype(np.int64), code)
    f, ex = np.frexp(np.where(small, 1.0, a))         # a = f * 2^ex, f in [0.5, 1)
    e = ex - 1                                          # a = (2f) * 2^e, 2f in [1, 2)
    q = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    normal_code = ((e + 7) << 3) | q
    code = np.where(small, code, normal_code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg & ~nan, 0x80, 0)
    return code.astype(np.uint8)


def quantize_per_tensor(x):
    """(codes uint8, descale float32) for one tensor, per the recipe above.

    ``x`` holds the tensor's values exactly in float32 (bf16 inputs upcast).
    """
    x = np.asarray(x, dtype=np.float32)
    absmax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    s = np.float32(np.maximum(absmax, SCALE_FLOOR)) / np.float32(E4M3_MAX)
    s = np.float32(s)
    qv = (x / s).astype(np.float32)
    return e4m3_encode_rne_sat(qv), s

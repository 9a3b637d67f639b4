"""Number formats the oracle reads -- test infrastructure only.

* bf16: the upper 16 bits of an IEEE binary32; widening is exact.
* e4m3: the OCP 8-bit "E4M3FN" format -- 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals at exponent field 0, no infinities, and
  NaN only at S.1111.111, so the largest finite magnitude is 448. The pages
  name an FP8 forward path without a format (page "r/mlscaling", FA3 bullet);
  E4M3FN is the plainest reading of "e4m3" and the format gfx950 multiplies.
* per-tensor quantisation: amax over the whole tensor, codes are the e4m3
  round-to-nearest-even of x * (448 / amax) computed in float32, and the
  descale is amax / 448 in float32 (1 when amax is 0). The scale product is
  done in float32 because it decides an integer code, and float32 is the
  precision the kernel uses for it.

The decode table is built from the format definition above, not from any
library; ``tests/test_codecs.py`` pins it against torch's float8_e4m3fn.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E, ascending in value as in code.
_POS = E4M3_TABLE[:0x7F]


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode e4m3 codes (uint8) to float64 by table lookup."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(x) -> np.ndarray:
    """Round to the nearest e4m3 value, ties to the even code, saturating at +-448.

    Works on magnitudes: finds the two table neighbours of |x| and keeps the
    closer one; an exact tie keeps the code whose mantissa LSB (code bit 0)
    is zero. The sign bit is copied from x (so -0.0 encodes as 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("f64_to_e4m3: NaN input")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS[hi], hi, code).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def quantize_per_tensor(x):
    """Per-tensor amax quantisation of a float32 tensor to e4m3.

    Returns (codes uint8 with x's shape, descale float32) such that
    decode(codes) * descale approximates x.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return f64_to_e4m3(x.astype(np.float64)), np.float32(1.0)
    s = np.float32(E4M3_MAX) / amax
    xs = (x * s).astype(np.float32)
    return f64_to_e4m3(xs.astype(np.float64)), np.float32(amax / np.float32(E4M3_MAX))


def dequantize(codes, descale) -> np.ndarray:
    """Float64 values the FP8 kernel multiplies: decode(code) * descale."""
    return e4m3_to_f64(codes) * np.float64(np.float32(descale))

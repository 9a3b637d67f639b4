"""The e4m3 forward's emulated exponential (CPU): its constants against what they are stated to do.

The kernel (csrc/fwd.hip) encodes p * 112 = 2^t as the byte round(8 t + 56 - kCodeShift) on unmasked tiles
(round to nearest even, negatives clamped to 0: the byte conversion's behaviour). Here the constants are read
from the source and the encoding is evaluated in float64 against the e4m3 decoding of the oracle's codec: the
code stays a finite e4m3 value wherever the rescale threshold allows (t <= log2 448), its decoded value is
within the stated error of 2^t, and the shift makes the ratio average 1 over the fractional part of t.
"""
import math
import os
import re

import numpy as np

from oracle import codecs

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tiled_online_softmax_amd", "csrc",
                   "fwd.hip")


def _constant(name):
    m = re.search(rf"constexpr\s+(?:float|int)\s+{name}\s*=\s*([0-9.eE+-]+)f?;", open(SRC).read())
    assert m, name
    return float(m.group(1))


SHIFT, TAU, LOG112 = _constant("kCodeShift"), _constant("kTauP8"), _constant("kLog2P8")
DECODE = codecs.e4m3_to_f64(np.arange(256, dtype=np.uint8))


def _code(t):
    x = 8.0 * np.asarray(t, dtype=np.float64) + 56.0 - SHIFT
    return np.clip(np.rint(x), 0, 255).astype(np.int64)  # np.rint rounds half to even


def test_constants():
    assert LOG112 == np.float32(math.log2(112))
    assert 112 * 2.0 ** TAU == 448.0  # the largest p the encoding must hold is 2^tau


def test_codes_stay_finite_up_to_the_threshold():
    t = np.linspace(-12.0, math.log2(448.0), 200001)
    c = _code(t)
    assert c.max() <= 126 and np.all(np.isfinite(DECODE[c]))  # 0x7E = 448; 0x7F is NaN in e4m3fn
    assert _code(-7.2) == 0 and _code(-1e30) == 0  # far below the reference max: p encodes as 0


def test_decoded_error_and_mean():
    t = (np.arange(400000) + 0.5) / 400000 * 8.0 - 2.0  # eight octaves in the normal range, uniform fractions
    ratio = DECODE[_code(t)] / np.exp2(t)
    assert 0.92 < ratio.min() and ratio.max() < 1.066  # -7.9% ... +6.5%
    assert abs(ratio.mean() - 1.0) < 2e-4  # the shift centres the chord
    assert math.sqrt(np.mean((ratio - 1.0) ** 2)) < 0.032  # rms 3.1%
    rne = DECODE[codecs.f64_to_e4m3(np.exp2(t))] / np.exp2(t)  # round-to-nearest of the exact value, for scale
    assert math.sqrt(np.mean((rne - 1.0) ** 2)) < 0.027


def test_code_is_monotone():
    t = np.linspace(-7.0, math.log2(448.0), 100001)
    assert np.all(np.diff(DECODE[_code(t)]) >= 0)

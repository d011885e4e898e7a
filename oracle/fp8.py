"""OCP 8-bit floating point, E4M3 variant ("e4m3fn") -- oracle codec.

TEST INFRASTRUCTURE ONLY: this module belongs to the CPU oracle.  Only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library.

The pages say only that the lightning indexer runs in FP8 ("Paper Breakdown:
DeepSeek-V3.2", section 2 "Architecture: DSA (§2.1)", the note under the
index-score formula; "DeepSeek-V3.2: Pushing the Frontier of Open Large
Language Models", Key points, first bullet).  The variant used here is the
OCP E4M3 format that gfx950 implements natively, written out from the
format definition:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 encodes subnormals  (-1)^s * (m/8) * 2^-6;
* otherwise                            (-1)^s * (1 + m/8) * 2^(e-7);
* there are no infinities; S.1111.111 (0x7F, 0xFF) is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448 and the smallest subnormal is 2^-9.

Encoding rounds to the nearest representable value, ties to the even
mantissa, after clamping to [-448, 448]; NaN encodes to 0x7F.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_SUBNORMAL = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 e4m3fn codes to float64, straight from the field layout."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = np.ldexp(m / 8.0, -6)
    nrm = np.ldexp(1.0 + m / 8.0, np.maximum(e, 1) - 7)
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# The 127 non-negative finite values, indexed by their code 0x00..0x7E.  The
# code order is the value order, so "even code" is "even mantissa".
_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Encode float values to e4m3fn codes: clamp, round to nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.clip(np.abs(np.where(nan, 0.0, x)), 0.0, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_POS_VALUES[hi] == a, hi, code)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def dequantize(codes, scale) -> np.ndarray:
    """Value of a scaled FP8 tensor: scale * decode(code), in float64.

    ``scale`` broadcasts over the trailing (feature) dimension.
    """
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def quantize_rows(x):
    """Per-row FP8 quantisation of float32 rows ``x[..., d]``.

    One float32 scale per row maps the row's largest magnitude onto the
    largest e4m3fn value: scale = amax / 448 (float32 division, correctly
    rounded), or 1 for a row of zeros; each element becomes
    encode(x / scale), the quotient again a correctly rounded float32.  The
    pages fix only that the indexer runs in FP8 ("Paper Breakdown:
    DeepSeek-V3.2", section 2 "Architecture: DSA (§2.1)", the note under the
    index-score formula); the per-token amax/448 scale is the reading used
    for every FP8 operand here.  Rows must be finite.

    Returns (codes uint8 [..., d], scale float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(y.astype(np.float64)), scale

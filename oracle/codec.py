"""Oracle codec for 8-bit floating point, E4M3 with no infinities ("e4m3fn").

Test infrastructure only (see the package docstring).

The pages leave FP8 rounding open ("RedFuser episode transcript", cues 33 and
61: the quantisation case study is real-number algebra and the text does not
say how FP8 rounding is done). The reading taken, the plainest one consistent
with a largest code of 448: the OCP 8-bit E4M3 format -- 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
m * 2^-9; the code with all exponent and mantissa bits set is NaN; there is no
infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. Encoding rounds
to the nearest representable value, ties to the code with an even mantissa,
after clamping the magnitude to 448 (saturation).

The encoder is a nearest-value search over the table of all finite codes built
from that definition, so it can be checked by eye. Parity: pinned by an
exhaustive round trip of all 254 finite codes, by the rounding of hand-picked
ties, and by torch's CPU float8_e4m3fn cast inside the finite range.
"""

import numpy as np


def _code_value(code):
    """Value of one non-negative code 0..126 from the format definition."""
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


_POS_VALUES = np.array([_code_value(c) for c in range(127)], dtype=np.float64)


def e4m3_table():
    """Values of the non-negative finite codes 0x00..0x7E, ascending."""
    return _POS_VALUES.copy()


def e4m3_decode(codes):
    """uint8 codes -> float64 values (0x7F and 0xFF decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag_code = c & 0x7F
    val = np.where(mag_code == 0x7F, np.nan, _POS_VALUES[np.minimum(mag_code, 126)])
    return np.where(c & 0x80, -val, val)


def e4m3_encode(x):
    """Finite float values -> uint8 codes, round to nearest, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode expects finite inputs")
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), _POS_VALUES[-1])
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # _POS_VALUES[hi] >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    exact = d_hi == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact | pick_hi, hi, lo).astype(np.uint8)
    return np.where(sign, code | 0x80, code).astype(np.uint8)

"""Number formats of the KV cache: E4M3 (FP8) and E2M1 (FP4).

"DeepSeek-V4.1 架构解析" §03: the main KV is stored as MXFP4 -- E2M1 values with an E4M3 scale per 16
channels -- and the SWA KV stays in FP8.  The page's range argument
(448 x 6 = 2688) fixes the E4M3 variant: the largest finite value is 448, i.e.
the "FN" variant (no infinities; exponent 15 / mantissa 7 is NaN), and the
largest E2M1 magnitude is 6.

Encoding is written as "nearest value of the finite value set, ties to the code
whose last mantissa bit is 0", which is IEEE round-to-nearest-even restated for
a small table, with saturation to the largest finite magnitude (the method
never produces NaN).  The sign bit is the sign bit of the input, as in an IEEE
conversion, so small negative values encode to negative zero.
"""

import numpy as np

# ---------------------------------------------------------------- E4M3 (FN) --


def _e4m3_value(b):
    """Value of E4M3FN bytes (int array), by the format's definition.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
    Exponent 0 is subnormal: m/8 * 2**-6.  Byte 0x7F / 0xFF is NaN.
    """
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# The definition applied once to each of the 256 bytes; decoding a large
# array is then one table lookup per byte.
_E4M3_TABLE = _e4m3_value(np.arange(256))


def e4m3_decode(b):
    """Decode E4M3FN bytes to float64 (see _e4m3_value for the layout)."""
    return _E4M3_TABLE[np.asarray(b, dtype=np.uint8)]


# All non-negative finite E4M3FN magnitudes, indexed by their byte (0x00..0x7E).
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
E4M3_MAX = float(_E4M3_POS[-1])  # 448


def _round_to_table(mag, table):
    """Index of the nearest table value to each |x|; ties go to the even index.

    ``table`` is sorted ascending and its index is the code, so "even index"
    is "last mantissa bit 0".  Magnitudes above the last entry saturate.
    """
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(table, mag, side="left")  # first table[i] >= mag
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= table[-1], len(table) - 1, idx)
    return idx


def e4m3_encode(x):
    """Round float values to E4M3FN bytes: RNE, saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    code = _round_to_table(np.abs(x), _E4M3_POS).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


# ------------------------------------------------------------------- E2M1 --

# E2M1: 2 exponent bits (bias 1), 1 mantissa bit; code 0..7 magnitudes.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = float(E2M1_VALUES[-1])  # 6


def e2m1_decode(c):
    """Decode 4-bit E2M1 codes (bit 3 = sign) to float64."""
    c = np.asarray(c).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where((c >> 3) & 1, -mag, mag)


def e2m1_encode(x):
    """Round float values to 4-bit E2M1 codes: RNE, saturating at +-6."""
    x = np.asarray(x, dtype=np.float64)
    code = _round_to_table(np.abs(x), E2M1_VALUES).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 3
    return (code | sign).astype(np.uint8)

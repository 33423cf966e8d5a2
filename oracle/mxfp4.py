"""MXFP4 KV-cache entries: E2M1 values with one E4M3 scale per 16 channels.

"DeepSeek-V4.1 架构解析" §03 fixes the format (E2M1 elements, an E4M3 scale per 16 channels, no
second-level/global scale) and that quantization happens after RoPE and only
for storage (entries are dequantized before attention).

Readings where the page is silent:
  * scale rule: s = RNE_E4M3(amax / 6), saturating at 448, so the largest
    element of a group maps near the E2M1 maximum 6 (the page's 448 x 6 = 2688
    range argument);
  * a scale that rounds to 0 (amax / 6 <= 2**-10) gives all-zero magnitudes;
  * element rule: code = signbit(x) << 3 | RNE_E2M1(|x| / s), saturating at 6
    (|x| / s can exceed 6 because s was rounded);
  * byte layout of one 512-channel entry: 256 code bytes, channel 2k in the low
    nibble of byte k and channel 2k+1 in the high nibble, plus a separate plane
    of 32 scale bytes (one per 16-channel group, in channel order).

The divisions amax / 6 and |x| / s are done in float64.  They decide the same
rounding as exact real division: x is float32 (24-bit significand) and s, 6 and
every E2M1/E4M3 rounding midpoint have at most 5 significant bits, so a
quotient that is not exactly a midpoint differs from one by at least ~2**-24
relative, far more than float64's 2**-53 rounding error.
"""

import numpy as np

from .formats import e4m3_decode, e4m3_encode, e2m1_decode, e2m1_encode

GROUP = 16  # channels per E4M3 scale


def quantize(x):
    """Quantize float32 entries [..., D] (D a multiple of 32) to MXFP4.

    Returns (codes uint8 [..., D/2], scales uint8 [..., D/16]).
    """
    x = np.asarray(x)
    assert x.dtype == np.float32, "the quantizer input is the float32 post-RoPE entry"
    d = x.shape[-1]
    assert d % (2 * GROUP) == 0
    g = x.astype(np.float64).reshape(x.shape[:-1] + (d // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)
    scale_bytes = e4m3_encode(amax / 6.0)
    s = e4m3_decode(scale_bytes)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s > 0, np.abs(g) / np.where(s > 0, s, 1.0), 0.0)
    mag_codes = e2m1_encode(ratio) & 7
    sign = np.signbit(g).astype(np.uint8) << 3
    codes4 = (mag_codes | sign).reshape(x.shape[:-1] + (d,))
    packed = (codes4[..., 0::2] | (codes4[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_bytes.astype(np.uint8)


def unpack_codes(codes):
    """Packed bytes [..., D/2] -> 4-bit codes [..., D] in channel order."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def dequantize(codes, scales):
    """MXFP4 entries back to float64 values s * E2M1(c) (exact)."""
    c = unpack_codes(codes)
    v = e2m1_decode(c)
    s = e4m3_decode(scales)
    d = c.shape[-1]
    v = v.reshape(v.shape[:-1] + (d // GROUP, GROUP)) * s[..., None]
    return v.reshape(v.shape[:-2] + (d,))

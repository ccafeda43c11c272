"""OCP FP8 E4M3FN format model — TEST INFRASTRUCTURE ONLY.

[FA3-wiki] "Nuevas capacidades de hardware de la GPU Hopper" and innovation 3
name 8-bit floating point with a limited dynamic range; the pages do not fix
the encoding. Reading used here: the OCP 8-bit floating point "E4M3FN"
format, one sign bit, 4 exponent bits with bias 7 and 3 mantissa bits:

* exponent field 0: subnormal, value = m/8 · 2^−6 (step 2^−9);
* exponent field 1..15: value = (1 + m/8) · 2^(e−7);
* the codes with all of exponent and mantissa set (0x7F, 0xFF) are NaN, so
  the largest finite magnitude is 1.75 · 2^8 = 448; there is no infinity.

Encoding rounds to nearest with ties to the even code (the code whose
mantissa's last bit is 0) and saturates: any finite magnitude ≥ 448 encodes
as ±448. NaN inputs are not expected and are rejected.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code):
    """Value of an 8-bit code (int or integer array), NaN for 0x7F/0xFF."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_values():
    """Magnitudes of the non-negative finite codes 0x00..0x7E, increasing."""
    return e4m3_decode(np.arange(0x7F))


_POS = None


def e4m3_encode(x):
    """Round-to-nearest-even, saturating encode of float64 values to codes.

    Returns uint8 codes. The nearest of the 127 finite magnitudes is chosen;
    an exact tie picks the even code. Zero (of either sign) encodes as +0.
    """
    global _POS
    if _POS is None:
        _POS = e4m3_values()
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN cannot be encoded")
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, mag, side="left")          # first value >= mag
    hi = np.clip(hi, 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_hi = _POS[hi] - mag
    d_lo = mag - _POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.int64)
    neg = (x < 0) & (code != 0)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)

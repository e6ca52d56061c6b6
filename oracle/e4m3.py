"""OCP E4M3FN decode (D) and encode (E) — oracle, test infrastructure only.

Source: "ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section "Design" item 3
(activations are encoded to OCP e4m3 with round-to-nearest-even and saturation, so that a
row-sum of decoded codes is exact by construction) and section "hardware e4m3 convert in the
producers" (the encoder maps NaN to 0 and -0 to +0 and clamps to +-448 before rounding).

Format (OCP 8-bit floating point, E4M3FN): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits. Exponent field 0 is subnormal: value = m * 2^-9. 0x7F / 0xFF are NaN; there is no
infinity. Largest finite magnitude 0x7E = 448.

Reading taken where the page is silent: a negative input whose magnitude rounds to zero keeps
its sign (code 0x80); only an exact -0.0 input becomes 0x00. Both decode to zero, so neither
changes any sum.
"""
import numpy as np

MAX_FINITE = 448.0
NAN_CODES = (0x7F, 0xFF)


def _decode_one(code: int) -> float:
    """Value of one E4M3FN code, from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


#: D: float64 value of every code 0..255 (NaN for 0x7F and 0xFF).
DECODE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

#: the 127 non-negative finite magnitudes, ascending; index == code for codes 0x00..0x7E.
_MAGS = DECODE[:0x7F].copy()
assert np.all(np.diff(_MAGS) > 0)
#: midpoints between neighbouring magnitudes (exact dyadic numbers in fp64).
_MIDS = (_MAGS[:-1] + _MAGS[1:]) / 2.0


def decode(codes) -> np.ndarray:
    """D: codes (uint8 array) -> float64 values."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(q) -> np.ndarray:
    """E: float32 array -> uint8 E4M3FN codes.

    NaN -> 0x00; exact -0.0 -> 0x00; otherwise the sign bit is kept, |q| is clamped to 448
    (so +-inf -> +-448) and rounded to the nearest representable magnitude, ties going to
    the code whose least significant bit is 0.
    """
    q = np.asarray(q, dtype=np.float32)
    a = np.abs(q.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, MAX_FINITE))
    # idx = number of midpoints strictly below a  -> candidate code when a is not a midpoint
    lo = np.searchsorted(_MIDS, a, side="left")   # midpoints < a
    hi = np.searchsorted(_MIDS, a, side="right")  # midpoints <= a
    tie = hi != lo                                 # a is exactly the midpoint between codes lo, lo+1
    code = np.where(tie, np.where(lo % 2 == 0, lo, lo + 1), lo).astype(np.uint8)
    neg = np.signbit(q) & ~nan
    neg_zero = neg & (q == 0)
    code = np.where(neg & ~neg_zero, code | 0x80, code).astype(np.uint8)
    return code


def nearest_magnitudes(a: float):
    """Brute-force helper for pins: every finite non-negative code whose value is nearest to
    ``a`` (a >= 0, finite, <= 448), by exhaustive search over the table."""
    d = np.abs(_MAGS - a)
    return np.flatnonzero(d == d.min())

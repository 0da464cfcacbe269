"""Brute-force E4M3 helpers used only to pin the oracle.

Built from the field definition with exact rationals and an exhaustive
search over all finite codes, so they share no arithmetic with
``oracle.e4m3`` (which uses frexp / ldexp / rint).
"""

from fractions import Fraction

import numpy as np


def frac_decode(code):
    """Exact value of one E4M3 code as a Fraction (None for NaN)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        mag = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        mag = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
    return -mag if s else mag


FINITE_POS_CODES = [c for c in range(0x7F)]             # 0x00..0x7E
FINITE_POS_VALUES = np.array([float(frac_decode(c)) for c in FINITE_POS_CODES])


def nearest_even_code(x):
    """Exhaustive nearest-even encode of float64 values (|x| <= 448 expected).

    Distances to every finite positive code are exact in fp64 for the inputs
    used (bf16 values times powers of two); ties go to the code whose
    mantissa LSB is 0; the sign bit follows the input's sign (so a negative
    value that rounds to zero gives 0x80); magnitudes above 448 give 0x7E.
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    a = np.abs(x)
    d = np.abs(a[:, None] - FINITE_POS_VALUES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.array(FINITE_POS_CODES)
    even = (codes & 1) == 0
    pick_even = cand & even[None, :]
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    mag = codes[idx]
    mag = np.where(a > 448.0, 0x7E, mag)
    sign = np.signbit(x).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def all_finite_bf16_bits(max_abs=None):
    """Every finite bf16 bit pattern, optionally with |value| <= max_abs."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits.astype(np.uint32) >> 7) & 0xFF
    bits = bits[exp != 0xFF]
    if max_abs is not None:
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        bits = bits[np.abs(vals) <= max_abs]
    return bits


def bf16_value(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

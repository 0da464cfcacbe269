"""Brute-force E2M1 helpers used only to pin the oracle.

Built from the field definition with exact rationals and an exhaustive
search over the eight magnitudes, so they share no arithmetic with
``oracle.e2m1`` (which uses frexp / ldexp / rint).
"""

from fractions import Fraction

import numpy as np


def frac_decode(code):
    """Exact value of one E2M1 nibble as a Fraction."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0:
        mag = Fraction(m, 2)
    else:
        mag = (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -mag if s else mag


POS_CODES = list(range(8))
POS_VALUES = np.array([float(frac_decode(c)) for c in POS_CODES])


def nearest_even_code(x):
    """Exhaustive nearest-even E2M1 encode of float64 values; ties go to the
    code whose mantissa bit is 0, the sign follows the input, magnitudes
    above 6 give 6."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    a = np.abs(x)
    d = np.abs(a[:, None] - POS_VALUES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.array(POS_CODES)
    pick_even = cand & ((codes & 1) == 0)[None, :]
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    mag = np.where(a > 6.0, 7, codes[idx])
    return (mag | (np.signbit(x).astype(np.int64) << 3)).astype(np.uint8)


def smallest_exponent(amax, top=6):
    """Smallest integer e with max(amax, 1e-4) <= top * 2^e, by exact
    rational search (amax a float; 1e-4 taken as its float64 value)."""
    a = max(Fraction(float(amax)), Fraction(float(np.float64(1e-4))))
    e = 0
    while a > top * Fraction(2) ** e:
        e += 1
    while a <= top * Fraction(2) ** (e - 1):
        e -= 1
    return e

"""OCP 8-bit floating point, E4M3 variant (no infinities; 0x7F / 0xFF are NaN).

The pages only say the indexer K cache holds "FP8" codes (IndexCache blog
post, the "FP8 naive cache" snippet: 128 bytes of K plus a 4-byte fp32
scale).  The reading adopted here is the OCP E4M3 format, largest finite
value 448:

  byte b = s eeee mmm
  e == 0            ->  (-1)^s * m * 2^-9             (subnormal; m == 0 is a signed zero)
  e == 15, m == 7   ->  NaN
  otherwise         ->  (-1)^s * (1 + m/8) * 2^(e-7)

Encoding rounds to the nearest representable value, ties to the even code
(mantissa LSB 0), keeps the sign of results that round to zero, and
saturates magnitudes above 448 to 448.  TEST INFRASTRUCTURE ONLY.
"""

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
QUANTUM_SUBNORMAL_EXP = -9  # subnormal spacing 2^-9
CODE_MAX_FINITE = 0x7E


def decode(codes):
    """Decode uint8 E4M3 codes to float64 (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    subnormal = np.ldexp(m.astype(np.float64), -9)
    mag = np.where(e == 0, subnormal, normal)
    val = np.where(sign == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val


def encode(x):
    """Encode float64 values to E4M3 codes: round to nearest, ties to even.

    For |x| >= 2^-6 with binade [2^j, 2^(j+1)) the spacing of E4M3 values is
    2^(j-3); below 2^-6 it is the subnormal spacing 2^-9.  ``n`` is x counted
    in those quanta, rounded half-to-even; the code is then the binade's base
    code plus n (a carry into the next binade falls out of the arithmetic).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("e4m3.encode: non-finite input")
    neg = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    j = ex.astype(np.int64) - 1            # floor(log2 a) for a > 0
    sub = a < MIN_NORMAL
    qexp = np.where(sub, QUANTUM_SUBNORMAL_EXP, j - 3)
    n = np.rint(np.ldexp(a, -qexp))        # exact scaling, then half-to-even
    mag = np.where(sub, n, (j + 6) * 8 + n)
    mag = np.minimum(mag, CODE_MAX_FINITE).astype(np.int64)
    return (mag | (neg << 7)).astype(np.uint8)

"""OCP 4-bit float E2M1 and the 8-bit power-of-two scale E8M0.
TEST INFRASTRUCTURE ONLY.

The pages name an FP4 variant of the indexer K cache (IndexCache blog post,
the ``use_fp4_cache`` argument that ``SparseAttnIndexer.forward_cuda`` passes
to the op) but give no format.  The reading adopted is the element type and
the scale type of the OCP Microscaling (MX) formats, version 1.0 (its FP4
element and its E8M0 shared scale), which gfx950's scaled matrix cores take
as operands directly:

  nibble c = s ee m
  e == 0   ->  (-1)^s * m * 2^-1                 (0 or 0.5; m == 0 is a signed zero)
  e  > 0   ->  (-1)^s * (1 + m/2) * 2^(e-1)      (1, 1.5, 2, 3, 4, 6)
  no infinities, no NaN.

  E8M0 byte u -> 2^(u - 127); u = 255 is NaN (never produced here).

Encoding rounds to the nearest representable value, ties to the even code
(m = 0), keeps the sign of a result that rounds to zero and saturates
magnitudes above 6 to 6.
"""

import numpy as np

MAX_FINITE = 6.0
MIN_NORMAL = 1.0
QUANTUM_SUBNORMAL_EXP = -1   # subnormal spacing 2^-1
CODE_MAX_FINITE = 0x7
E8M0_BIAS = 127


def decode(codes):
    """Decode E2M1 nibbles (0..15, any integer dtype) to float64 (exact)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("e2m1.decode: codes are 4-bit")
    sign = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp(1.0 + m / 2.0, e - 1)
    subnormal = np.ldexp(m.astype(np.float64), QUANTUM_SUBNORMAL_EXP)
    mag = np.where(e == 0, subnormal, normal)
    return np.where(sign == 1, -mag, mag)


def encode(x):
    """Encode float64 values to E2M1 nibbles (uint8 0..15): nearest, ties to even.

    In the binade [2^j, 2^(j+1)) (j >= 0) the spacing is 2^(j-1); below 1 it
    is the subnormal spacing 2^-1.  ``n`` counts x in those quanta, rounded
    half-to-even; the code is the binade's base code plus n, where a carry
    into the next binade falls out of the arithmetic.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("e2m1.encode: non-finite input")
    neg = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    j = ex.astype(np.int64) - 1            # floor(log2 a) for a > 0
    sub = a < MIN_NORMAL
    qexp = np.where(sub, QUANTUM_SUBNORMAL_EXP, j - 1)
    n = np.rint(np.ldexp(a, -qexp))        # exact scaling, then half-to-even
    mag = np.where(sub, n, 2 * j + n)      # binade j starts at code 2(j+1) = 2j + 2 quanta
    mag = np.minimum(mag, CODE_MAX_FINITE).astype(np.int64)
    return (mag | (neg << 3)).astype(np.uint8)


def e8m0_value(u):
    """E8M0 bytes -> float64 powers of two (NaN for 255)."""
    u = np.asarray(u).astype(np.int64)
    return np.where(u == 255, np.nan, np.ldexp(1.0, u - E8M0_BIAS))

"""Pins for the oracle's E4M3 codec (CPU only)."""

import json
import math
import os

import numpy as np

from oracle import e4m3
from tests.fp8_bruteforce import (all_finite_bf16_bits, bf16_value, frac_decode,
                                  nearest_even_code)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_table.json")


def _parse(v):
    if v == "nan":
        return math.nan
    if v == "-0":
        return -0.0
    return float(eval(v.replace("^", "**"), {"__builtins__": {}}))


def test_decode_matches_ocp_table():
    table = json.load(open(GOLDEN))["values"]
    for row in table:
        code = int(row["code"], 16)
        want = _parse(row["value"])
        got = float(e4m3.decode(np.array([code], np.uint8))[0])
        if math.isnan(want):
            assert math.isnan(got), row
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), row


def test_decode_all_codes_exact_rationals():
    codes = np.arange(256, dtype=np.uint8)
    got = e4m3.decode(codes)
    for c in range(256):
        f = frac_decode(c)
        if f is None:
            assert np.isnan(got[c])
        else:
            assert got[c] == float(f)


def test_decode_structure():
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                          # strictly increasing
    neg = e4m3.decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)                         # sign symmetry
    # equal spacing inside each binade, doubling from one binade to the next
    for e in range(1, 15):
        vals = pos[e * 8:(e + 1) * 8]
        assert np.all(np.diff(vals) == vals[1] - vals[0])
        assert np.array_equal(pos[(e + 1) * 8:(e + 2) * 8][:7 if e == 14 else 8],
                              (2 * vals)[:7 if e == 14 else 8])


def test_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = e4m3.encode(e4m3.decode(codes))
    assert np.array_equal(back, codes)


def test_encode_midpoints_go_to_even():
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = e4m3.encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got.astype(np.int64), want)
    assert np.array_equal(e4m3.encode(-mids).astype(np.int64), want | 0x80)


def test_encode_matches_bruteforce_on_all_bf16():
    bits = all_finite_bf16_bits(max_abs=448.0)
    x = bf16_value(bits)
    assert x.size > 30000
    assert np.array_equal(e4m3.encode(x), nearest_even_code(x))


def test_encode_scaled_bf16_matches_bruteforce():
    # bf16 values divided by powers of two, as the quantiser produces them
    rng = np.random.default_rng(7)
    bits = rng.choice(all_finite_bf16_bits(max_abs=448.0), 4000)
    for s in (-12, -3, 0, 2, 4):
        x = np.ldexp(bf16_value(bits), s)
        x = x[np.abs(x) <= 448]
        assert np.array_equal(e4m3.encode(x), nearest_even_code(x))


def test_encode_signed_zero_and_saturation():
    assert e4m3.encode(np.array([0.0]))[0] == 0x00
    assert e4m3.encode(np.array([-0.0]))[0] == 0x80
    assert e4m3.encode(np.array([-1e-30]))[0] == 0x80
    assert e4m3.encode(np.array([2.0 ** -10]))[0] == 0x00    # exact half of min subnormal -> even (0)
    assert e4m3.encode(np.array([3 * 2.0 ** -10]))[0] == 0x02
    assert e4m3.encode(np.array([1e6]))[0] == 0x7E
    assert e4m3.encode(np.array([-1e6]))[0] == 0xFE

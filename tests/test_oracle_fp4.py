"""Pins for the oracle's FP4 indexer K cache (CPU only): the E2M1 / E8M0
codec against the OCP MX table and an exhaustive rational search, the
per-32 quantiser against exact rational exponents and codes, the byte
layout against hand-placed bytes, and the score against exact rationals and
against the FP8 cache's score on rows both caches hold exactly."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import Batch, e2m1, e4m3, fp4cache, logits, paged
from tests.fp4_bruteforce import frac_decode, nearest_even_code, smallest_exponent
from tests.fp8_bruteforce import all_finite_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_ocp_table.json")


def _parse(v):
    if v == "nan":
        return math.nan
    if v == "-0":
        return -0.0
    return float(eval(v.replace("^", "**"), {"__builtins__": {}}))


def _bf16(x):
    """float values -> bf16 bit patterns (round to nearest even)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


# ------------------------------------------------------------------ codec --

def test_decode_matches_ocp_table():
    table = json.load(open(GOLDEN))
    for row in table["e2m1"]:
        got = float(e2m1.decode(np.array([int(row["code"], 16)]))[0])
        want = _parse(row["value"])
        assert got == want and math.copysign(1, got) == math.copysign(1, want), row
    for row in table["e8m0"]:
        got = float(e2m1.e8m0_value(np.array([int(row["code"], 16)]))[0])
        want = _parse(row["value"])
        assert (math.isnan(got) and math.isnan(want)) or got == want, row


def test_decode_all_codes_exact_rationals():
    got = e2m1.decode(np.arange(16))
    for c in range(16):
        assert got[c] == float(frac_decode(c))
    assert np.all(np.diff(got[:8]) > 0)
    assert np.array_equal(got[8:], -got[:8])


def test_encode_roundtrip_every_code():
    for c in range(16):
        v = e2m1.decode(np.array([c]))
        assert int(e2m1.encode(v)[0]) == c


def test_encode_dense_sweep_and_midpoints():
    grid = np.arange(-8 * 256, 8 * 256 + 1) / 256.0            # every multiple of 2^-8 in [-8, 8]
    mids = (e2m1.decode(np.arange(7)) + e2m1.decode(np.arange(1, 8))) / 2
    eps = np.array([0.0, 2.0 ** -40, -(2.0 ** -40)])
    near = (mids[:, None] + eps[None, :]).reshape(-1)
    x = np.concatenate([grid, near, -near, [-0.0, 1e-30, -1e-30, 6.5, 1e9, -1e9]])
    assert np.array_equal(e2m1.encode(x), nearest_even_code(x))


@pytest.mark.parametrize("e", [-15, -3, 0, 4, 60, 126])
def test_encode_every_bf16_value_at_a_scale(e):
    """Each finite bf16 value scaled by 2^-e and kept where the quantiser could
    see it (|x| <= 6 * 2^e): the oracle's code equals the exhaustive search."""
    bits = all_finite_bf16_bits()
    x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = x[np.abs(x) <= np.ldexp(6.0, e)]
    y = np.ldexp(x, -e)
    assert np.array_equal(e2m1.encode(y), nearest_even_code(y))


# -------------------------------------------------------------- quantiser --

def test_group_exponent_exact():
    rng = np.random.default_rng(31)
    vals = np.concatenate([
        np.ldexp(6.0, np.arange(-20, 120)),                    # on a boundary: e exactly k
        np.nextafter(np.ldexp(6.0, np.arange(-20, 120)), np.inf),
        np.nextafter(np.ldexp(6.0, np.arange(-20, 120)), 0),
        np.abs(rng.standard_normal(300)) * np.ldexp(1.0, rng.integers(-30, 100, 300)),
        [0.0, 1e-4, 9e-5, 1.1e-4, 3.3e38],
    ])
    got = fp4cache.group_exponent(vals)
    for v, g in zip(vals, got):
        assert g == smallest_exponent(v), v


def _rows(seed, n):
    """bf16 rows whose four groups have different magnitudes, with special groups."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 4, 32)) * np.ldexp(1.0, rng.integers(-12, 12, (n, 4, 1)))
    x[0] = 0.0                                   # all-zero row: the floor exponent
    x[1, 2] = 0.0                                # one zero group
    x[2, 1, :] = 0.0
    x[2, 1, 5] = -6.0 * 2 ** 3                   # amax exactly 6 * 2^3
    x[3, 3] *= 1e-30                             # bf16-subnormal group
    x[4, 0, ::2] = 1e-8                          # tiny values that round to (signed) zero
    x[4, 0, 1::2] = -1e-8
    return _bf16(x.reshape(n, 128))


def test_quantize_rows_against_exact_search():
    bits = _rows(32, 40)
    codes, e = fp4cache.quantize_rows(bits)
    x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 4, 32)
    for r in range(x.shape[0]):
        for g in range(4):
            want_e = smallest_exponent(np.abs(x[r, g]).max())
            assert e[r, g] == want_e, (r, g)
            want = nearest_even_code(np.ldexp(x[r, g], -want_e))
            assert np.array_equal(codes[r, 32 * g:32 * (g + 1)], want), (r, g)
    assert e[0].tolist() == [-15] * 4 and not codes[0].any()
    assert e[2, 1] == 3 and codes[2, 32 + 5] == 0xF     # -6 * 2^3 -> code -6


def test_dequantize_error_bound():
    """|x - dequant| is at most half the spacing at |x|'s binade, never more than 2^e."""
    bits = _rows(33, 60)
    codes, e = fp4cache.quantize_rows(bits)
    x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    back = fp4cache.dequantize(codes, e)
    ee = np.repeat(e, 32, axis=1)
    y = np.abs(np.ldexp(x, -ee))
    spacing = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    assert np.all(np.abs(x - back) <= np.ldexp(spacing / 2, ee))
    assert np.all(np.abs(back) <= np.ldexp(6.0, ee))


# ----------------------------------------------------------------- layout --

def test_layout_hand_placed_bytes():
    """Position 17 of block 2 with one nonzero value, 3.0 at dim 32*2 + 7
    (group 2, byte 3, high nibble): group 2's amax 3 gives e = -1 (3 <= 6 *
    2^-1) and the code of 3 / 2^-1 = 6, 0x7; the other groups are all zero
    (floor exponent -15).  Exactly the position's 64 code bytes and 4 scale
    bytes are written."""
    cache = fp4cache.new_cache(4, fill=0xEE)
    row = np.zeros(128, np.float32)
    row[64 + 7] = 3.0
    fp4cache.quant_write_k(cache, _bf16(row)[None, :], [2 * 64 + 17])
    blk = cache[2]
    for g in range(4):
        codes = blk[g * 1024 + 17 * 16:g * 1024 + 18 * 16]
        want = np.zeros(16, np.uint8)
        if g == 2:
            want[3] = 0x70
        assert codes.tolist() == want.tolist(), g
        # scale byte 4096 + g*64 + (17 % 16)*4 + 17 // 16
        assert blk[4096 + g * 64 + 5] == (-1 if g == 2 else -15) + 127, g
    changed = set(np.nonzero(cache.reshape(-1) != 0xEE)[0].tolist())
    expect = {2 * 4352 + g * 1024 + 17 * 16 + i for g in range(4) for i in range(16)}
    expect |= {2 * 4352 + 4096 + g * 64 + 5 for g in range(4)}
    assert changed == expect


def test_write_read_roundtrip_and_skips():
    rng = np.random.default_rng(34)
    bits = _rows(35, 50)
    slots = rng.permutation(6 * 64)[:50]
    slots[7] = -1
    cache = fp4cache.new_cache(6, fill=0xEE)
    fp4cache.quant_write_k(cache, bits, slots)
    codes, e = fp4cache.quantize_rows(bits)
    bt = np.arange(6)
    keep = slots >= 0
    got = fp4cache.read_tokens(cache, bt, slots[keep])
    assert np.array_equal(got, fp4cache.dequantize(codes[keep], e[keep]))
    # untouched slots keep their fill bytes
    untouched = np.setdiff1d(np.arange(6 * 64), slots[keep])
    for s in untouched[:20]:
        b, p = divmod(int(s), 64)
        assert np.all(cache[b, fp4cache.code_offsets([p])[0]] == 0xEE)
        assert np.all(cache[b, fp4cache.scale_offsets([p])[0]] == 0xEE)


def test_offsets_tile_the_block():
    """The code and scale bytes of the 64 positions cover the 4352-byte block once."""
    p = np.arange(64)
    offs = np.concatenate([fp4cache.code_offsets(p).reshape(-1), fp4cache.scale_offsets(p).reshape(-1)])
    assert np.array_equal(np.sort(offs), np.arange(fp4cache.BLOCK_BYTES))


# ------------------------------------------------------------------ score --

FINITE8 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _fp4_case(seed, H, S, T, spread=6):
    rng = np.random.default_rng(seed)
    nib = rng.integers(0, 16, (S, 128)).astype(np.uint8)
    e = rng.integers(-spread, spread + 1, (S, 4))
    q8 = rng.choice(FINITE8, (T, H, 128))
    w = rng.standard_normal((T, H)).astype(np.float32)
    nb = -(-S // 64)
    bt = rng.permutation(nb + 3)[:nb]
    cache = fp4cache.new_cache(nb + 3, fill=0xEE)
    slots = bt[np.arange(S) // 64] * 64 + np.arange(S) % 64
    fp4cache.write_tokens(cache, slots, nib, e)
    return nib, e, q8, w, cache, Batch([S], [0, T], bt[None, :])


def test_logits_match_exact_rationals():
    from tests.fp8_bruteforce import frac_decode as f8
    for seed, H, S, T in [(41, 3, 70, 2), (42, 2, 20, 3)]:
        nib, e, q8, w, cache, batch = _fp4_case(seed, H, S, T)
        got = fp4cache.logits(q8, w, cache, batch)
        for t in range(T):
            p = batch.token_position(t)
            for s in range(p + 1):
                total = Fraction(0)
                for h in range(H):
                    d = Fraction(0)
                    for j in range(128):
                        d += f8(int(q8[t, h, j])) * frac_decode(int(nib[s, j])) * Fraction(2) ** int(e[s, j // 32])
                    if d > 0:
                        total += Fraction(float(w[t, h])) * d
                assert abs(got[t][s] - float(total)) <= 1e-12 * max(1.0, abs(float(total)))


def test_logits_equal_fp8_cache_on_shared_rows():
    """Rows whose four group exponents are equal hold values that an FP8 row
    with scale 2^e holds exactly (every E2M1 value is an E4M3 value): the two
    caches' scores agree bit for bit."""
    rng = np.random.default_rng(43)
    S, H, T = 150, 8, 3
    nib = rng.integers(0, 16, (S, 128)).astype(np.uint8)
    er = rng.integers(-8, 4, S)
    e = np.repeat(er[:, None], 4, axis=1)
    q8 = rng.choice(FINITE8, (T, H, 128))
    w = rng.standard_normal((T, H)).astype(np.float32)
    nb = -(-S // 64)
    bt = rng.permutation(nb + 2)[:nb]
    slots = bt[np.arange(S) // 64] * 64 + np.arange(S) % 64
    c4 = fp4cache.new_cache(nb + 2)
    fp4cache.write_tokens(c4, slots, nib, e)
    c8 = paged.new_cache(nb + 2, 64)
    codes8 = e4m3.encode(e2m1.decode(nib))
    assert np.array_equal(e4m3.decode(codes8), e2m1.decode(nib))
    paged.write_tokens(c8, slots, codes8, np.ldexp(1.0, er).astype(np.float32))
    batch = Batch([S], [0, T], bt[None, :])
    got4 = fp4cache.logits(q8, w, c4, batch)
    got8 = logits.logits(q8, w, c8, batch)
    for t in range(T):
        assert np.array_equal(got4[t], got8[t])

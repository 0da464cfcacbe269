"""Pins for the oracle's quantiser, cache layout and weight fold (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, paged, quant
from synth import f32_to_bf16_bits
from tests.fp8_bruteforce import all_finite_bf16_bits, bf16_value, nearest_even_code


def _smallest_e_bruteforce(a):
    """Linear search with exact rationals: smallest e with max(a,1e-4) <= 448*2^e."""
    a = max(Fraction(a), Fraction(1e-4))
    e = -200
    while a > 448 * Fraction(2) ** e:
        e += 1
    return e


def test_ue8m0_bruteforce_sample():
    rng = np.random.default_rng(1)
    bits = rng.choice(all_finite_bf16_bits(), 300)
    a = np.abs(bf16_value(bits))
    e = quant.ue8m0_exponent(a)
    for ai, ei in zip(a, e):
        assert ei == _smallest_e_bruteforce(ai)


def test_ue8m0_invariants_all_positive_bf16():
    bits = all_finite_bf16_bits()
    a = np.abs(bf16_value(bits))
    e = quant.ue8m0_exponent(a)
    fl = np.maximum(a, 1e-4)
    assert np.all(fl <= np.ldexp(448.0, e))
    assert np.all(fl > np.ldexp(448.0, e - 1))
    big = a >= 1e-4
    ratio = a[big] / np.ldexp(1.0, e[big])
    assert np.all((ratio > 224) & (ratio <= 448))


def test_quantize_rows_elementwise_bruteforce():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[3] *= 1e-3
    x[4] *= 300.0
    bits = f32_to_bf16_bits(x)
    codes, scale = quant.quantize_rows(bits)
    sc = scale.astype(np.float64)
    # scale is an exact power of two (fp32 mantissa bits all zero)
    assert np.all((scale.view(np.uint32) & 0x7FFFFF) == 0)
    xv = bf16_value(bits)
    want = nearest_even_code((xv / sc[:, None]).reshape(-1)).reshape(codes.shape)
    assert np.array_equal(codes, want)
    # reconstruction error within half a quantum of the E4M3 grid
    rec = e4m3.decode(codes) * sc[:, None]
    y = np.abs(xv / sc[:, None])
    quantum = np.where(y < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, np.floor(np.log2(np.maximum(y, 1e-300))).astype(int) - 3))
    assert np.all(np.abs(rec - xv) <= 0.5 * quantum * sc[:, None])
    # the largest element of each row lands in [224, 448] (amax/scale is in
    # (224, 448] before rounding, and 224 is itself a code)
    amax_code = np.abs(e4m3.decode(codes)).max(axis=1)
    assert np.all((amax_code >= 224) & (amax_code <= 448))


def test_quantize_special_rows():
    zero = np.zeros((1, 128), np.uint16)
    codes, scale = quant.quantize_rows(zero)
    assert np.all(codes == 0) and scale[0] == np.float32(2.0 ** -22)
    negzero = np.full((1, 128), 0x8000, np.uint16)
    codes, scale = quant.quantize_rows(negzero)
    assert np.all(codes == 0x80) and scale[0] == np.float32(2.0 ** -22)
    tiny = f32_to_bf16_bits(np.full((1, 128), 1e-6, np.float32))
    codes, scale = quant.quantize_rows(tiny)
    assert scale[0] == np.float32(2.0 ** -22)
    assert np.all(codes == nearest_even_code(bf16_value(tiny) * 2.0 ** 22))
    # amax exactly 448 * 2^k gives scale 2^k; one bf16 step above gives 2^(k+1)
    row = np.zeros((2, 128), np.float32)
    row[0, 5] = 448.0 * 4
    row[1, 5] = np.float32(448.0 * 4 * (1 + 2 ** -7))
    codes, scale = quant.quantize_rows(f32_to_bf16_bits(row))
    assert scale[0] == 4.0 and codes[0, 5] == 0x7E
    assert scale[1] == 8.0


def test_cache_layout_hand_computed():
    # block_size 2: a block is 2*128 code bytes then 2*4 scale bytes (264 bytes)
    cache = paged.new_cache(num_blocks=3, block_size=2, fill=0xA5)
    codes = np.arange(128, dtype=np.uint8)
    paged.write_token(cache, slot=3, codes=codes, scale=np.float32(2.0 ** -7))
    flat = cache.reshape(-1)
    # slot 3 = block 1, offset 1 -> codes at 264 + 128, scale at 264 + 256 + 4
    assert np.array_equal(flat[392:520], codes)
    assert bytes(flat[524:528]) == np.float32(2.0 ** -7).tobytes()   # 00 00 00 3c
    assert bytes(flat[524:528]) == b"\x00\x00\x00\x3c"
    untouched = np.ones(flat.size, bool)
    untouched[392:520] = False
    untouched[524:528] = False
    assert np.all(flat[untouched] == 0xA5)


def test_scatter_is_a_bijection_and_skips_padding():
    nb, bs = 5, 64
    rng = np.random.default_rng(3)
    cache = paged.new_cache(nb, bs, fill=0xA5)
    x = rng.standard_normal((nb * bs, 128)).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    slots = rng.permutation(nb * bs)
    quant.quant_write_k(cache, bits, slots)
    codes, scale = quant.quantize_rows(bits)
    # read back every slot and compare with what was written there
    inv = np.empty_like(slots)
    inv[slots] = np.arange(slots.size)
    bt = np.arange(nb)
    got_c, got_s = paged.read_tokens(cache, bt, np.arange(nb * bs))
    assert np.array_equal(got_c, codes[inv])
    assert np.array_equal(got_s, scale[inv].astype(np.float64))
    # padding rows (slot -1) change nothing
    before = cache.copy()
    quant.quant_write_k(cache, bits[:4], np.array([-1, -1, -1, -1]))
    assert np.array_equal(before, cache)


def test_partial_scatter_leaves_other_bytes():
    cache = paged.new_cache(4, 64, fill=0x5A)
    rng = np.random.default_rng(4)
    bits = f32_to_bf16_bits(rng.standard_normal((10, 128)).astype(np.float32))
    slots = np.array([0, 63, 64, 100, 127, 128, 200, 255, -1, 17])
    quant.quant_write_k(cache, bits, slots)
    written = np.zeros(cache.size, bool)
    for s in slots[slots >= 0]:
        b, off = divmod(int(s), 64)
        written[b * 8448 + off * 128: b * 8448 + off * 128 + 128] = True
        written[b * 8448 + 8192 + off * 4: b * 8448 + 8192 + off * 4 + 4] = True
    assert np.all(cache.reshape(-1)[~written] == 0x5A)


def test_fold_closed_form():
    w = np.ones((2, 64), np.float32)
    qs = np.full((2, 64), 2.0 ** -7, np.float32)
    out = quant.fold_weights(w, qs)
    # powers of two are exact, so the result is 2^-10 * fp32(128^-0.5)
    assert np.all(out == np.float32(2.0 ** -10) * np.float32(0.08838834764831845))
    w2 = np.array([[3.0] * 64], np.float32)
    out2 = quant.fold_weights(w2, np.ones((1, 64), np.float32))
    assert np.allclose(out2, 3.0 * 128 ** -0.5 / 8, rtol=1e-6)


@pytest.mark.parametrize("shape", [(3, 64, 128)])
def test_quantize_q_per_head(shape):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(shape).astype(np.float32)
    x[1, 7] *= 50
    q8, qs = quant.quantize_q(f32_to_bf16_bits(x))
    assert q8.shape == shape and qs.shape == shape[:2]
    # each (token, head) row has its own scale: the scaled-up head gets a larger one
    assert qs[1, 7] > 8 * np.median(qs)


def test_write_tokens_equals_token_by_token():
    """The many-token scatter places every byte exactly as write_token does,
    and leaves every other byte alone."""
    rng = np.random.default_rng(5)
    nb, bs = 9, 64
    a = paged.new_cache(nb, bs, fill=0xEE)
    b = paged.new_cache(nb, bs, fill=0xEE)
    slots = rng.permutation(nb * bs)[:200]
    codes = rng.integers(0, 256, (200, 128), dtype=np.uint8)
    scales = np.ldexp(1.0, rng.integers(-20, 10, 200)).astype(np.float32)
    for s_, c, sc in zip(slots, codes, scales):
        paged.write_token(a, s_, c, sc)
    paged.write_tokens(b, slots, codes, scales)
    assert np.array_equal(a, b)
    assert np.count_nonzero(a != 0xEE) <= 200 * 132

"""Pins for the oracle's lightning-indexer scores (CPU only)."""

from fractions import Fraction

import numpy as np

from oracle import Batch, e4m3, logits, paged
from tests.fp8_bruteforce import frac_decode

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _paged_setup(rng, codes, scales, block_size=64, spare=3):
    """Write logical K (codes [S,128], scales [S]) into a shuffled pool."""
    S = codes.shape[0]
    nb = -(-S // block_size)
    pool = nb + spare
    bt = rng.permutation(pool)[:nb]
    cache = paged.new_cache(pool, block_size, fill=0xEE)
    for s in range(S):
        slot = bt[s // block_size] * block_size + s % block_size
        paged.write_token(cache, slot, codes[s], scales[s])
    return cache, bt


def _random_case(seed, H, S, T):
    rng = np.random.default_rng(seed)
    kc = rng.choice(FINITE, (S, 128))
    ks = np.ldexp(1.0, rng.integers(-9, -5, S)).astype(np.float32)
    q8 = rng.choice(FINITE, (T, H, 128))
    w = rng.standard_normal((T, H)).astype(np.float32)
    cache, bt = _paged_setup(rng, kc, ks)
    batch = Batch([S], [0, T], bt[None, :])
    return kc, ks, q8, w, cache, batch


def _bruteforce(q8_t, w_t, kc, ks, p):
    """Exact rational evaluation of the definition, loop by loop."""
    H = q8_t.shape[0]
    out = []
    for s in range(p + 1):
        total = Fraction(0)
        for h in range(H):
            d = Fraction(0)
            for j in range(128):
                d += frac_decode(int(q8_t[h, j])) * frac_decode(int(kc[s, j]))
            if d > 0:
                total += Fraction(float(w_t[h])) * d
        out.append(total * Fraction(float(ks[s])))
    return out


def test_logits_match_exact_rationals():
    for seed, H, S, T in [(11, 4, 40, 2), (12, 2, 70, 1), (13, 3, 9, 9)]:
        kc, ks, q8, w, cache, batch = _random_case(seed, H, S, T)
        got = logits.logits(q8, w, cache, batch)
        for t in range(T):
            p = batch.token_position(t)
            want = _bruteforce(q8[t], w[t], kc, ks, p)
            assert got[t].shape == (p + 1,)
            for g, wv in zip(got[t], want):
                assert abs(g - float(wv)) <= 1e-12 * max(1.0, abs(float(wv)))


def _code(v):
    return int(e4m3.encode(np.array([v]))[0])


def test_hand_computed_case():
    # two heads reading one dimension each; K rows chosen so each head's dot
    # product is a known number; ReLU applies per head before the weighting
    S = 3
    kc = np.zeros((S, 128), np.uint8)
    kc[0, 3], kc[0, 7] = _code(2.0), _code(-1.0)     # head0: 2, head1: -1
    kc[1, 3], kc[1, 7] = _code(-4.0), _code(0.5)     # head0: -4, head1: 0.5
    kc[2, 3], kc[2, 7] = _code(1.5), _code(3.0)      # head0: 1.5, head1: 3
    ks = np.array([2.0 ** -7, 2.0 ** -6, 1.0], np.float32)
    q8 = np.zeros((1, 2, 128), np.uint8)
    q8[0, 0, 3] = _code(1.0)
    q8[0, 1, 7] = _code(1.0)
    w = np.array([[0.5, -2.0]], np.float32)
    cache, bt = _paged_setup(np.random.default_rng(0), kc, ks)
    got = logits.logits(q8, w, cache, Batch([S], [0, 1], bt[None, :]))[0]
    # token 0 of a request with 3 positions and 1 new token -> p = 2
    want = [(0.5 * 2.0 + 0.0) * 2.0 ** -7,
            (0.0 + (-2.0) * 0.5) * 2.0 ** -6,
            (0.5 * 1.5 + (-2.0) * 3.0) * 1.0]
    assert np.array_equal(got, np.array(want))


def test_causal_range_includes_self():
    kc, ks, q8, w, cache, batch = _random_case(21, 2, 65, 5)
    got = logits.logits(q8, w, cache, batch)
    for t in range(5):
        assert got[t].shape == (65 - 5 + t + 1,)


def test_invariants():
    kc, ks, q8, w, cache, batch = _random_case(31, 8, 130, 3)
    base = logits.logits(q8, w, cache, batch)
    # w >= 0  =>  I >= 0
    pos = logits.logits(q8, np.abs(w), cache, batch)
    assert all(np.all(v >= 0) for v in pos.values())
    # scaling w by 2^j scales I exactly; negating w negates I
    sc = logits.logits(q8, w * np.float32(8.0), cache, batch)
    ng = logits.logits(q8, -w, cache, batch)
    for t in base:
        assert np.array_equal(sc[t], base[t] * 8.0)
        assert np.array_equal(ng[t], -base[t])
    # permuting heads (q rows with their weights) changes nothing
    perm = np.random.default_rng(1).permutation(8)
    ph = logits.logits(q8[:, perm], w[:, perm], cache, batch)
    for t in base:
        assert np.allclose(ph[t], base[t], rtol=1e-13, atol=0)
    # weights are linear: I(w1 + w2) = I(w1) + I(w2)
    w2 = np.random.default_rng(2).standard_normal(w.shape).astype(np.float32)
    a = logits.logits(q8, w2, cache, batch)
    b = logits.logits(q8, (w + w2).astype(np.float32), cache, batch)
    for t in base:
        assert np.allclose(b[t], base[t] + a[t], rtol=1e-5, atol=1e-9 * np.abs(base[t]).max())


def test_paging_invariance():
    rng = np.random.default_rng(41)
    S = 200
    kc = rng.choice(FINITE, (S, 128))
    ks = np.ldexp(1.0, rng.integers(-9, -5, S)).astype(np.float32)
    q8 = rng.choice(FINITE, (2, 4, 128))
    w = rng.standard_normal((2, 4)).astype(np.float32)
    c1, bt1 = _paged_setup(np.random.default_rng(1), kc, ks)
    c2, bt2 = _paged_setup(np.random.default_rng(2), kc, ks, spare=9)
    assert not np.array_equal(bt1, bt2[:bt1.size])
    r1 = logits.logits(q8, w, c1, Batch([S], [0, 2], bt1[None, :]))
    r2 = logits.logits(q8, w, c2, Batch([S], [0, 2], bt2[None, :]))
    for t in r1:
        assert np.array_equal(r1[t], r2[t])


def test_relu_zeroes_negative_heads():
    # q = -k for every head: every dot product is -|k|^2 < 0, so I == 0
    rng = np.random.default_rng(51)
    kc = rng.choice(FINITE[FINITE < 0x7F], (4, 128))     # non-negative codes
    kc[:, 0] = _code(1.0)
    ks = np.ones(4, np.float32)
    cache, bt = _paged_setup(rng, kc, ks)
    q8 = np.zeros((1, 3, 128), np.uint8)
    q8[0, :, :] = kc[3] | 0x80                           # negated last K row
    w = np.array([[1.0, -1.0, 2.0]], np.float32)
    got = logits.logits(q8, w, cache, Batch([4], [0, 1], bt[None, :]))[0]
    assert got[3] == 0.0

"""The FP4 indexer K cache: quantiser, byte layout, scatter, gather and
scores.  TEST INFRASTRUCTURE ONLY.

The pages only name the variant (IndexCache blog post: ``use_fp4_cache`` in
``SparseAttnIndexer.forward_cuda``).  Everything below is the reading
adopted for it; each choice keeps the FP8 cache's conventions where one
carries over.

Quantiser (per K row of 128 bf16 values):
  * four groups of 32 consecutive dims, g = d // 32, each with its own
    power-of-two scale 2^e_g (the MX block size of 32, E8M0 scale);
  * e_g = the smallest integer with max(amax_g, 1e-4) <= 6 * 2^e_g, the
    FP8 cache's ue8m0 rule with E2M1's largest value 6 in place of 448, so
    no code saturates;
  * code = E2M1 encode of x / 2^e_g (nearest, ties to even, sign kept).

Block of 64 positions (4352 bytes = 64 * 68: half the FP8 cache's 128 code
bytes plus four scale bytes per position):
  codes   byte g*1024 + p*16 + i          dims 32g+2i (bits 0-3) and 32g+2i+1
                                          (bits 4-7) of position p
  scales  byte 4096 + g*64 + (p%16)*4 + p//16
                                          E8M0 byte e_g + 127 of position p
Slot s lives in block s // 64 at position s % 64, as in the FP8 cache.

Score (the FP8 cache's score with K decoded group by group):
  I[t, s] = sum_h w[t, h] * max(0, sum_d q8[t, h, d] * c[s, d] * 2^e[s, d // 32])
with c the decoded E2M1 values; no separate per-position scale remains.
"""

import numpy as np

from . import e2m1, e4m3
from .quant import AMAX_FLOOR, bf16_to_f64

HEAD_DIM = 128
GROUP = 32
GROUPS = HEAD_DIM // GROUP
BLOCK = 64
CODE_BYTES = BLOCK * HEAD_DIM // 2          # 4096
BLOCK_BYTES = CODE_BYTES + BLOCK * GROUPS   # 4352


def group_exponent(amax):
    """Smallest integer e with max(amax, 1e-4) <= 6 * 2^e (exact comparisons)."""
    a = np.maximum(np.asarray(amax, dtype=np.float64), AMAX_FLOOR)
    _, ex = np.frexp(a / e2m1.MAX_FINITE)         # first guess, then fix up exactly
    e = ex.astype(np.int64)
    while True:
        low = a > np.ldexp(e2m1.MAX_FINITE, e)
        if not low.any():
            break
        e = e + low
    while True:
        high = a <= np.ldexp(e2m1.MAX_FINITE, e - 1)
        if not high.any():
            break
        e = e - high
    return e


def quantize_rows(x_bits):
    """Rows of 128 bf16 values -> (codes uint8 [..., 128] nibbles, e int64 [..., 4])."""
    x = bf16_to_f64(x_bits)
    if x.shape[-1] != HEAD_DIM:
        raise ValueError("rows must hold 128 values")
    g = x.reshape(x.shape[:-1] + (GROUPS, GROUP))
    e = group_exponent(np.abs(g).max(axis=-1))
    codes = e2m1.encode(np.ldexp(g, -e[..., None]))
    return codes.reshape(x.shape), e


def dequantize(codes, e):
    """codes [..., 128], e [..., 4] -> float64 values [..., 128]."""
    c = e2m1.decode(codes).reshape(np.shape(codes)[:-1] + (GROUPS, GROUP))
    return np.ldexp(c, np.asarray(e, dtype=np.int64)[..., None]).reshape(np.shape(codes))


def new_cache(num_blocks, fill=0):
    return np.full((num_blocks, BLOCK_BYTES), fill, dtype=np.uint8)


def code_offsets(p):
    """[n, 64] byte offsets (within a block) of positions p's code bytes, by
    group then byte: entry 16g + i is g*1024 + p*16 + i."""
    p = np.asarray(p, dtype=np.int64).reshape(-1, 1)
    g = np.arange(GROUPS).repeat(16)[None, :]
    i = np.tile(np.arange(16), GROUPS)[None, :]
    return g * 1024 + p * 16 + i


def scale_offsets(p):
    """[n, 4] byte offsets of positions p's scale bytes, group by group."""
    p = np.asarray(p, dtype=np.int64).reshape(-1, 1)
    g = np.arange(GROUPS)[None, :]
    return CODE_BYTES + g * 64 + (p % 16) * 4 + p // 16


def pack_codes(codes):
    """Nibbles [n, 128] -> bytes [n, 64] (dim 2i in bits 0-3, dim 2i+1 in bits 4-7)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], HEAD_DIM), np.uint8)
    out[:, 0::2] = b & 15
    out[:, 1::2] = b >> 4
    return out


def write_tokens(cache, slots, codes, e):
    """Store rows (nibbles [n,128], exponents [n,4]) at distinct slots >= 0."""
    slots = np.asarray(slots, dtype=np.int64)
    if slots.size == 0:
        return
    b, p = slots // BLOCK, slots % BLOCK
    cache[b[:, None], code_offsets(p)] = pack_codes(codes)
    cache[b[:, None], scale_offsets(p)] = (np.asarray(e, dtype=np.int64) + e2m1.E8M0_BIAS).astype(np.uint8)


def read_tokens(cache, block_table_row, positions):
    """Decoded K values [n, 128] (float64) of logical positions of one request."""
    positions = np.asarray(positions, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[positions // BLOCK]
    p = positions % BLOCK
    codes = unpack_codes(cache[blocks[:, None], code_offsets(p)])
    e = cache[blocks[:, None], scale_offsets(p)].astype(np.int64) - e2m1.E8M0_BIAS
    return dequantize(codes, e)


def quant_write_k(cache, k_bits, slot_mapping):
    """Quantise each K row and store it at its slot; slot < 0 is skipped (the
    FP8 path's op-body scatter, ``ops.indexer_k_quant_and_cache``)."""
    k_bits = np.asarray(k_bits, dtype=np.uint16).reshape(-1, HEAD_DIM)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if slots.shape[0] != k_bits.shape[0]:
        raise ValueError("one slot per K row")
    codes, e = quantize_rows(k_bits)
    keep = slots >= 0
    write_tokens(cache, slots[keep], codes[keep], e[keep])
    return cache


def logits_row(q8_t, w_t, cache, block_table_row, p):
    """I[t, 0..p] for one query token, fp64.

    The per-head dot products are exact in fp64 when a row's group
    exponents lie within 20 of each other (every product is a multiple of
    2^(min e - 10) below 2^(max e + 12), and 128 of them need fewer than 53
    bits); only the weighted head sum rounds.
    """
    q = e4m3.decode(q8_t).reshape(-1, HEAD_DIM)
    k = read_tokens(cache, block_table_row, np.arange(p + 1))
    d = q @ k.T
    w = np.asarray(w_t, dtype=np.float64).reshape(-1, 1)
    return (w * np.maximum(d, 0.0)).sum(axis=0)


def logits(q8, w, cache, batch, rows=None):
    """Scores {t: fp64 row of length p_t + 1} for the query tokens in ``rows``."""
    if rows is None:
        rows = range(batch.num_tokens)
    out = {}
    for t in rows:
        r = batch.token_request(t)
        out[int(t)] = logits_row(q8[t], w[t], cache, batch.block_table[r],
                                 batch.token_position(t))
    return out

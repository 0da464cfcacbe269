"""Per-128 fp8 quantisation with ue8m0 scales, cache scatter, q quantisation
and the weight fold.  TEST INFRASTRUCTURE ONLY.

Pages: IndexCache blog post -- the "FP8 naive cache" snippet (128 bytes of K
plus one 4-byte fp32 scale per token, so one scale per 128-wide block), the
op body (``ops.indexer_k_quant_and_cache(k, kv_cache, slot_mapping,
quant_block_size, scale_fmt)``: K is quantised and scattered to its slot),
and ``Indexer.forward`` (q quantised per token-group of 128 with
``use_ue8m0=True``; weights multiplied by q_scale, softmax_scale and
n_head^-0.5).

Readings where the pages are silent:
  * ue8m0 scale = the smallest power of two 2^e with amax <= 448 * 2^e
    (rounding the scale up never saturates a code);
  * amax is floored at 1e-4, so an all-zero row gets scale 2^-22;
  * the same quantiser is used for q (per token and head) and for K;
  * slot < 0 marks a padding token whose K is not written;
  * softmax_scale = head_dim^-0.5;
  * the fold runs in fp32, left to right, as on the fp32 weights tensor of
    the pages.
"""

import numpy as np

from . import e4m3, paged

AMAX_FLOOR = 1e-4
QUANT_BLOCK = 128


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def ue8m0_exponent(amax):
    """Smallest integer e with max(amax, 1e-4) <= 448 * 2^e (exact comparisons)."""
    a = np.maximum(np.asarray(amax, dtype=np.float64), AMAX_FLOOR)
    _, ex = np.frexp(a / e4m3.MAX_FINITE)        # first guess, then fix up exactly
    e = ex.astype(np.int64)
    while True:
        too_small = a > np.ldexp(e4m3.MAX_FINITE, e)
        if not too_small.any():
            break
        e = e + too_small
    while True:
        can_lower = a <= np.ldexp(e4m3.MAX_FINITE, e - 1)
        if not can_lower.any():
            break
        e = e - can_lower
    return e


def quantize_rows(x_bits):
    """Quantise rows of 128 bf16 values.

    Returns (codes uint8 [..., 128], scale float32 [...]) with
    codes = encode(x / scale) and scale = 2^e, e = ue8m0_exponent(max|x|).
    Division by a power of two is an exact ldexp.
    """
    x = bf16_to_f64(x_bits)
    if x.shape[-1] != QUANT_BLOCK:
        raise ValueError("rows must hold 128 values")
    e = ue8m0_exponent(np.abs(x).max(axis=-1))
    codes = e4m3.encode(np.ldexp(x, -e[..., None]))
    scale = np.ldexp(np.ones_like(e, dtype=np.float64), e).astype(np.float32)
    return codes, scale


def quant_write_k(cache, k_bits, slot_mapping):
    """Quantise each K row and store it at its slot; slot < 0 is skipped.

    Mutates ``cache`` in place; bytes of all other slots are left unchanged.
    """
    k_bits = np.asarray(k_bits, dtype=np.uint16).reshape(-1, QUANT_BLOCK)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if slots.shape[0] != k_bits.shape[0]:
        raise ValueError("one slot per K row")
    codes, scale = quantize_rows(k_bits)
    keep = slots >= 0
    paged.write_tokens(cache, slots[keep], codes[keep], scale[keep])
    return cache


def quantize_q(q_bits):
    """q [T, H, 128] bf16 -> (q8 uint8 [T, H, 128], q_scale float32 [T, H])."""
    return quantize_rows(q_bits)


def fold_weights(w_raw, q_scale, head_dim=128):
    """w = w_raw * q_scale * softmax_scale * n_head^-0.5, in fp32, left to right.

    Follows the fold in ``Indexer.forward`` (IndexCache blog post).  n_head
    is the second dimension of ``w_raw``.
    """
    w = np.asarray(w_raw, dtype=np.float32)
    n_head = w.shape[-1]
    softmax_scale = np.float32(head_dim ** -0.5)
    head_norm = np.float32(n_head ** -0.5)
    out = w * np.asarray(q_scale, dtype=np.float32)
    out = out * softmax_scale
    out = out * head_norm
    return out.astype(np.float32)

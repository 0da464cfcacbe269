"""Byte layout of the paged indexer K cache.  TEST INFRASTRUCTURE ONLY.

The pages fix the cache tensor as uint8 of shape
``(num_blocks, block_size, head_dim + head_dim // quant_block_size * 4)``
(IndexCache blog post: ``DeepseekV32IndexerBackend.get_kv_cache_shape`` and
the "FP8 naive cache" snippet), i.e. 132 bytes per token for head_dim 128,
one shared K per position (``num_kv_heads == 1``), no V.

Reading (the pages give only the shape, not the byte order inside a
block): "block-split".  The ``block_size * 132`` bytes of block b are

  [0, block_size*128)                 the 128 code bytes of offsets 0..block_size-1
  [block_size*128, block_size*132)    the fp32 little-endian scales, 4 bytes each

so token (b, off) has codes at b*B + off*128 and its scale at
b*B + block_size*128 + off*4, with B = block_size*132.
"""

import numpy as np

HEAD_DIM = 128
TOKEN_BYTES = HEAD_DIM + 4


def block_bytes(block_size):
    return block_size * TOKEN_BYTES


def new_cache(num_blocks, block_size, fill=0):
    return np.full((num_blocks, block_size, TOKEN_BYTES), fill, dtype=np.uint8)


def _flat(cache):
    return cache.reshape(cache.shape[0], -1)


def slot_location(slot, block_size):
    """(block, offset) of a physical slot: slot = block * block_size + offset."""
    return slot // block_size, slot % block_size


def write_token(cache, slot, codes, scale):
    """Store 128 code bytes and one fp32 scale for the token at ``slot``."""
    block_size = cache.shape[1]
    b, off = slot_location(int(slot), block_size)
    flat = _flat(cache)
    flat[b, off * HEAD_DIM:(off + 1) * HEAD_DIM] = codes
    sb = np.frombuffer(np.float32(scale).astype("<f4").tobytes(), dtype=np.uint8)
    base = block_size * HEAD_DIM + off * 4
    flat[b, base:base + 4] = sb


def write_tokens(cache, slots, codes, scales):
    """write_token for many tokens at once: row i of ``codes`` and ``scales[i]``
    go to ``slots[i]`` (slots distinct, all >= 0).  The same byte placement as
    the per-token form, written with one fancy-indexed assignment per field."""
    block_size = cache.shape[1]
    slots = np.asarray(slots, dtype=np.int64)
    if slots.size == 0:
        return
    b, off = slots // block_size, slots % block_size
    flat = _flat(cache)
    flat[b[:, None], off[:, None] * HEAD_DIM + np.arange(HEAD_DIM)[None, :]] = codes
    sb = np.asarray(scales, dtype="<f4").reshape(-1).view(np.uint8).reshape(-1, 4)
    flat[b[:, None], block_size * HEAD_DIM + off[:, None] * 4 + np.arange(4)[None, :]] = sb


def read_tokens(cache, block_table_row, positions):
    """Codes [n,128] (uint8) and scales [n] (float64) of logical positions of one request.

    Logical position s lives in physical block ``block_table_row[s // block_size]``
    at offset ``s % block_size`` (the block-table indirection of the paged
    backend, IndexCache blog post, ``DeepseekV32IndexerCache``).
    """
    block_size = cache.shape[1]
    positions = np.asarray(positions, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[positions // block_size]
    offs = positions % block_size
    flat = _flat(cache)
    code_idx = offs[:, None] * HEAD_DIM + np.arange(HEAD_DIM)[None, :]
    codes = flat[blocks[:, None], code_idx]
    sidx = block_size * HEAD_DIM + offs[:, None] * 4 + np.arange(4)[None, :]
    sbytes = np.ascontiguousarray(flat[blocks[:, None], sidx])
    scales = sbytes.view("<f4").reshape(-1).astype(np.float64)
    return codes, scales

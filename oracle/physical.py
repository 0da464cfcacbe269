"""Logical -> physical top-k indices.  TEST INFRASTRUCTURE ONLY.

Page: vLLM API docs for ``vllm.v1.attention.backends.mla.index_group``,
``SparseMLAIndexGroup._convert_once``: the logical top-k of a token (request
positions) is turned once per index group into global cache slots through
the token's request, the block table and the block size, optionally with the
number of valid entries per row.

Readings (the conversion kernel itself is not printed):
  * slot = block_table[r][pos // block_size] * stride + pos % block_size,
    with stride = block_size unless a block stride in rows is given;
  * a -1 entry stays -1;
  * valid count of a row = its number of entries >= 0.
"""

import numpy as np


def to_physical(logical_rows, token_req, block_table, block_size, stride=None):
    """logical int32 [T, k] -> (physical int32 [T, k], valid counts int32 [T])."""
    lg = np.asarray(logical_rows, dtype=np.int64)
    stride = block_size if stride is None else stride
    out = np.full(lg.shape, -1, dtype=np.int64)
    for t in range(lg.shape[0]):
        r = int(token_req[t])
        for j in range(lg.shape[1]):
            pos = lg[t, j]
            if pos < 0:
                continue
            out[t, j] = block_table[r][pos // block_size] * stride + pos % block_size
    valid = (lg >= 0).sum(axis=1)
    return out.astype(np.int32), valid.astype(np.int32)

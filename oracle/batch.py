"""Batch metadata as the oracle sees it (host NumPy arrays).

Mirrors the fields of ``DeepseekV32IndexerMetadata`` on the IndexCache blog
post (seq_lens, slot_mapping, decode/prefill split) plus the per-request
block table the paged backend keeps (``DeepseekV32IndexerBackend``).
TEST INFRASTRUCTURE ONLY.

Reading (pages silent on where new tokens sit in a sequence): the
``n_r = query_start_loc[r+1] - query_start_loc[r]`` new tokens of request r
are its last n_r positions, so the i-th new token has absolute position
``p = seq_lens[r] - n_r + i`` and attends causally to positions 0..p
inclusive (its own K is written before scoring in the op body).
"""

import numpy as np


class Batch:
    def __init__(self, seq_lens, query_start_loc, block_table, block_size=64):
        self.seq_lens = np.asarray(seq_lens, dtype=np.int64)
        self.query_start_loc = np.asarray(query_start_loc, dtype=np.int64)
        self.block_table = np.asarray(block_table, dtype=np.int64)
        self.block_size = int(block_size)
        if self.query_start_loc.shape != (self.seq_lens.shape[0] + 1,):
            raise ValueError("query_start_loc must have num_reqs + 1 entries")
        if self.block_table.ndim != 2 or self.block_table.shape[0] != self.seq_lens.shape[0]:
            raise ValueError("block_table must be [num_reqs, width]")

    @property
    def num_reqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self):
        return int(self.query_start_loc[-1])

    def token_request(self, t):
        """Request index r with query_start_loc[r] <= t < query_start_loc[r+1]."""
        r = int(np.searchsorted(self.query_start_loc, t, side="right") - 1)
        if not (0 <= r < self.num_reqs) or t >= self.query_start_loc[r + 1]:
            raise IndexError(f"token {t} outside the batch")
        return r

    def token_position(self, t):
        """Absolute position p_t of query token t (see module docstring)."""
        r = self.token_request(t)
        n_r = self.query_start_loc[r + 1] - self.query_start_loc[r]
        return int(self.seq_lens[r] - n_r + (t - self.query_start_loc[r]))

    def positions(self):
        return np.array([self.token_position(t) for t in range(self.num_tokens)], dtype=np.int64)

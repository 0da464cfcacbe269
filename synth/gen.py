"""Seeded generators.  Random draws and batch / paging layout only.

Draw recipe (every stream is its own ``numpy.random.default_rng`` seeded by
``SeedSequence([seed, stream, layer, request])`` so any request of any layer
can be regenerated alone):

  stream 0  batch layout: sequence lengths (uniform integers in
            [len_lo, len_hi] unless fixed), then one permutation of the
            physical block pool whose first sum(ceil(L_r / 64)) entries are
            dealt to the requests in order (request 0 first)
  stream 1  K of request r in layer l: standard normal fp32 [L_r, 128] for
            positions 0..L_r-1, rounded to bf16 (nearest, ties to even)
  stream 2  q of layer l: standard normal fp32 [T, 64, 128] -> bf16
  stream 3  raw head weights of layer l: standard normal fp32 [T, 64]
  stream 4  planted positions of request r: ``planted`` distinct positions
            drawn uniformly from [0, L_r); their fp32 K rows are multiplied
            by 3 before the bf16 rounding (in every layer)

The last ``new_tokens`` positions of each request are this step's new
tokens; the others are cached context.
"""

import math

import numpy as np

from .configs import WorkloadSpec


def f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _rng(seed, stream, layer=0, req=0):
    return np.random.default_rng(np.random.SeedSequence([seed, stream, layer, req]))


class Workload:
    """Batch layout plus lazily drawn inputs of one synthetic workload."""

    def __init__(self, name, seed, seq_lens, new_tokens, block_table, num_blocks, k,
                 n_heads=64, head_dim=128, block_size=64, num_layers=1, pattern="F",
                 planted=0):
        self.name = name
        self.seed = int(seed)
        self.seq_lens = np.asarray(seq_lens, dtype=np.int32)
        nt = np.asarray(new_tokens, dtype=np.int64)
        if nt.ndim == 0:
            nt = np.full(self.seq_lens.shape[0], int(nt), dtype=np.int64)
        self.new_tokens = nt.astype(np.int32)
        self.query_start_loc = np.concatenate([[0], np.cumsum(nt)]).astype(np.int32)
        self.block_table = np.asarray(block_table, dtype=np.int32)
        self.num_blocks = int(num_blocks)
        self.k = int(k)
        self.n_heads = int(n_heads)
        self.head_dim = int(head_dim)
        self.block_size = int(block_size)
        self.num_layers = int(num_layers)
        self.pattern = pattern
        self.planted = int(planted)
        if np.any(self.new_tokens > self.seq_lens):
            raise ValueError("more new tokens than sequence length")

    # ---- layout -------------------------------------------------------
    @property
    def num_reqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self):
        return int(self.query_start_loc[-1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.num_reqs else 0

    @property
    def max_query_len(self):
        return int(self.new_tokens.max()) if self.num_reqs else 0

    def token_req(self):
        return np.repeat(np.arange(self.num_reqs), self.new_tokens).astype(np.int32)

    def token_pos(self):
        """Absolute position of every query token (new tokens are the last ones)."""
        out = []
        for r in range(self.num_reqs):
            L, n = int(self.seq_lens[r]), int(self.new_tokens[r])
            out.append(np.arange(L - n, L))
        return np.concatenate(out).astype(np.int64) if out else np.zeros(0, np.int64)

    def slots(self, r, positions):
        positions = np.asarray(positions, dtype=np.int64)
        blk = self.block_table[r].astype(np.int64)[positions // self.block_size]
        return blk * self.block_size + positions % self.block_size

    # ---- draws ----------------------------------------------------------
    def planted_positions(self, r):
        if self.planted == 0:
            return np.zeros(0, dtype=np.int64)
        g = _rng(self.seed, 4, 0, r)
        return np.sort(g.choice(int(self.seq_lens[r]), size=self.planted, replace=False))

    def request_k(self, layer, r):
        """bf16 bits [L_r, 128] of request r's K rows in ``layer``."""
        L = int(self.seq_lens[r])
        x = _rng(self.seed, 1, layer, r).standard_normal((L, self.head_dim), dtype=np.float32)
        hot = self.planted_positions(r)
        if hot.size:
            x[hot] *= np.float32(3.0)
        return f32_to_bf16_bits(x)

    def ctx_rows(self, layer, reqs=None):
        """Cached-context K rows and their slots: (bits [N, 128], slots int64 [N])."""
        reqs = range(self.num_reqs) if reqs is None else reqs
        ks, ss = [], []
        for r in reqs:
            L, n = int(self.seq_lens[r]), int(self.new_tokens[r])
            if L - n == 0:
                continue
            ks.append(self.request_k(layer, r)[: L - n])
            ss.append(self.slots(r, np.arange(L - n)))
        if not ks:
            return np.zeros((0, self.head_dim), np.uint16), np.zeros(0, np.int64)
        return np.concatenate(ks), np.concatenate(ss)

    def new_rows(self, layer):
        """This step's new K rows (one per query token, token order) and slots."""
        ks, ss = [], []
        for r in range(self.num_reqs):
            L, n = int(self.seq_lens[r]), int(self.new_tokens[r])
            if n == 0:
                continue
            ks.append(self.request_k(layer, r)[L - n:])
            ss.append(self.slots(r, np.arange(L - n, L)))
        if not ks:
            return np.zeros((0, self.head_dim), np.uint16), np.zeros(0, np.int64)
        return np.concatenate(ks), np.concatenate(ss)

    def q_bits(self, layer):
        x = _rng(self.seed, 2, layer).standard_normal(
            (self.num_tokens, self.n_heads, self.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(x)

    def w_raw(self, layer):
        return _rng(self.seed, 3, layer).standard_normal(
            (self.num_tokens, self.n_heads), dtype=np.float32)


def layout(seed, lengths, block_size, pool_factor):
    """Block table dealt from a seeded permutation of the physical pool."""
    g = _rng(seed, 0)
    nb = [math.ceil(int(L) / block_size) for L in lengths]
    total = sum(nb)
    pool = max(int(math.ceil(total * pool_factor)), total, 1)
    perm = g.permutation(pool)
    width = max(nb) if nb else 1
    bt = np.full((len(lengths), max(width, 1)), -1, dtype=np.int32)
    off = 0
    for r, n in enumerate(nb):
        bt[r, :n] = perm[off:off + n]
        off += n
    return bt, pool


def make_workload(spec: WorkloadSpec):
    g = _rng(spec.seed, 0, 0, 1)
    if spec.len_lo == spec.len_hi:
        lengths = np.full(spec.num_reqs, spec.len_lo, dtype=np.int64)
    else:
        lengths = g.integers(spec.len_lo, spec.len_hi + 1, size=spec.num_reqs)
    bt, pool = layout(spec.seed, lengths, spec.block_size, spec.pool_factor)
    return Workload(spec.name, spec.seed, lengths, spec.new_tokens, bt, pool, spec.k,
                    spec.n_heads, spec.head_dim, spec.block_size, spec.num_layers,
                    spec.pattern, spec.planted)


def random_batch(seed, lengths, new_tokens, k, block_size=64, pool_factor=1.5, name="custom",
                 planted=0, num_layers=1, pattern="F"):
    """A small custom workload (ragged lengths, arbitrary new-token counts)."""
    bt, pool = layout(seed, lengths, block_size, pool_factor)
    return Workload(name, seed, lengths, new_tokens, bt, pool, k, block_size=block_size,
                    planted=planted, num_layers=num_layers, pattern=pattern)

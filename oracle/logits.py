"""Lightning-indexer scores in fp64.  TEST INFRASTRUCTURE ONLY.

Definition (the DSA lightning indexer of DeepSeek-V3.2; the pages show its
inputs -- fp8 q of 64 heads sharing one fp8 K per position, and per-head
weights with q_scale, softmax_scale and n_head^-0.5 folded in, IndexCache
blog post ``Indexer.forward`` and ``SparseAttnIndexer.forward_cuda`` -- but
not the score itself, so this is the plainest reading consistent with
them):

    I[t, s] = ks[s] * sum_h  w[t, h] * max(0, sum_d q8[t, h, d] * k8[s, d])

for s in 0..p_t (causal, inclusive of the token's own position), where q8
and k8 are the decoded E4M3 values, ks[s] the fp32 scale stored with K at
position s, and w the folded fp32 weights passed in.  The q scale is not
applied here: it is already inside w (the ``forward_cuda`` snippet notes
q_scale is folded into the weights).

The per-head dot products are exact in fp64 (every product is a multiple of
2^-18 below 2^18, so partial sums of 128 of them need fewer than 53 bits);
only the weighted head sum rounds.
"""

import numpy as np

from . import e4m3, paged


def logits_row(q8_t, w_t, cache, block_table_row, p):
    """I[t, 0..p] for one query token (fp64 vector of length p + 1)."""
    q = e4m3.decode(q8_t).reshape(-1, paged.HEAD_DIM)        # [H, 128]
    codes, ks = paged.read_tokens(cache, block_table_row, np.arange(p + 1))
    k = e4m3.decode(codes)                                    # [n, 128]
    d = q @ k.T                                               # [H, n], exact
    w = np.asarray(w_t, dtype=np.float64).reshape(-1, 1)
    return (w * np.maximum(d, 0.0)).sum(axis=0) * ks


def logits(q8, w, cache, batch, rows=None):
    """Scores for the query tokens in ``rows`` (default: all).

    Returns a dict {t: fp64 vector of length p_t + 1}.
    """
    if rows is None:
        rows = range(batch.num_tokens)
    out = {}
    for t in rows:
        r = batch.token_request(t)
        p = batch.token_position(t)
        out[int(t)] = logits_row(q8[t], w[t], cache, batch.block_table[r], p)
    return out

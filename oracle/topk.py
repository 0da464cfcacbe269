"""Per-row top-k selection.  TEST INFRASTRUCTURE ONLY.

Pages: the shared ``topk_indices_buffer`` is int32 ``[max_num_batched_tokens,
index_topk]`` and entries that are not (yet) valid hold -1 (IndexCache blog
post: the op body resets rows to -1; the buffer-allocation snippet).

Readings where the pages are silent:
  * candidates of query token t are its causal positions 0..p_t;
  * ties are broken by the lower position;
  * -0.0 and +0.0 are equal scores;
  * a row lists its min(k, p_t + 1) selected positions in ascending
    position order, then -1 up to k.
"""

import numpy as np


def select(scores, k):
    """Positions of the k best scores: order by (-score, position), keep the first k.

    A stable full sort; returns the selected positions sorted ascending.
    """
    s = np.asarray(scores, dtype=np.float64)
    pos = np.arange(s.shape[0])
    order = np.lexsort((pos, -s))           # primary key -score, then position
    return np.sort(order[:min(k, s.shape[0])])


def topk_row(scores, k):
    """One output row of length k: selected positions ascending, then -1."""
    sel = select(scores, k)
    row = np.full(k, -1, dtype=np.int32)
    row[:sel.shape[0]] = sel
    return row


def topk(rows_scores, k):
    """{t: scores} -> {t: int32 row of length k}."""
    return {t: topk_row(s, k) for t, s in rows_scores.items()}


def kth_value(scores, k):
    """The k-th largest score of a row (the smallest selected one)."""
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    return s[min(k, s.shape[0]) - 1]

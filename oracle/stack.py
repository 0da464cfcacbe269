"""A stack of indexer layers under an IndexCache schedule.  TEST INFRASTRUCTURE ONLY.

Pages:
  * IndexCache blog post, the buffer-allocation snippet: one
    ``topk_indices_buffer`` tensor is handed to every decoder layer;
  * the MLA forward snippet: an F layer runs the indexer and refreshes the
    buffer, an S layer does not, so its sparse attention consumes what the
    most recent F layer left;
  * PR #37735 report, "Review highlights": no explicit hand-off, the
    persistent buffer carries the result.

Reading for K writes: by default every layer writes its new K rows into its
own cache (``write_k_on_s=True``); ``write_k_on_s=False`` is the pages'
variant in which S layers have no indexer and no K cache.
"""

import numpy as np

from . import logits as _logits
from . import quant, topk as _topk


def run_stack(layers, full, batch, k, rows=None, write_k_on_s=True):
    """Run the stack and return the buffer rows each layer consumes.

    ``layers``: list of dicts with keys cache, k_bits, slot_mapping, q8, w.
    ``full``: list of bools (F = True).  ``rows``: query tokens to score
    (default all).  Returns a list (one per layer) of {t: int32 row}.
    """
    if len(full) != len(layers):
        raise ValueError("one schedule entry per layer")
    if not full[0]:
        raise ValueError("layer 0 must be an F layer")
    buffer = None
    consumed = []
    for lay, is_f in zip(layers, full):
        if is_f or write_k_on_s:
            quant.quant_write_k(lay["cache"], lay["k_bits"], lay["slot_mapping"])
        if is_f:
            scores = _logits.logits(lay["q8"], lay["w"], lay["cache"], batch, rows)
            buffer = _topk.topk(scores, k)
        consumed.append({t: np.array(v, copy=True) for t, v in buffer.items()})
    return consumed

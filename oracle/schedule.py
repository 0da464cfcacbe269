"""IndexCache F/S layer schedule.  TEST INFRASTRUCTURE ONLY.

Pages:
  * IndexCache blog post, the ``skip_topk`` snippet: with no pattern a layer
    skips top-k iff ``max(layer_id - offset + 1, 0) % freq != 0`` (defaults
    freq 1, offset 2); with a pattern and ``0 <= layer_id < len(pattern)`` it
    skips iff ``pattern[layer_id] == "S"``.
  * PR #37735 report, "Key source snippets" (deepseek_v2.py): the schedule
    only applies when ``use_index_cache`` is set (default False), and its
    frequency form is written ``max(layer_id - 1, 0) % freq != 0``, which is
    the blog's form at the default offset 2.
  * PR #37735 report, "Risks & impact": the pattern length must equal the
    layer count and every character must be F or S.

Reading: a layer with no pattern entry (layer_id >= len(pattern)) keeps the
default, i.e. it is an F layer.  F = full (runs the indexer and refreshes the
shared top-k buffer), S = shared (reuses the buffer).
"""


def is_full(layer_id, use_index_cache=False, freq=1, pattern=None, offset=2):
    """True if layer ``layer_id`` computes top-k (an F layer)."""
    if not use_index_cache:
        return True
    if pattern is None:
        return max(layer_id - offset + 1, 0) % freq == 0
    if 0 <= layer_id < len(pattern):
        return pattern[layer_id] != "S"
    return True


def schedule(num_layers, use_index_cache=False, freq=1, pattern=None, offset=2):
    return [is_full(i, use_index_cache, freq, pattern, offset) for i in range(num_layers)]


def pattern_errors(pattern, num_layers):
    """Reasons a pattern is rejected (empty list = valid).

    Length and alphabet follow the PR report's risk note; "the first layer
    must be F" is this implementation's rule (no producer has written the
    buffer before layer 0).
    """
    errs = []
    if len(pattern) != num_layers:
        errs.append("length")
    if any(c not in "FS" for c in pattern):
        errs.append("alphabet")
    if len(pattern) > 0 and pattern[0] != "F":
        errs.append("first-layer-S")
    return errs

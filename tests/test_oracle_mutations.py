"""Plant plausible mistakes in the oracle (CPU only) and check a pin catches each.

Each mutant replaces one oracle function for the duration of one pin; the
pin must then fail.  Nothing here touches the GPU.
"""

import numpy as np
import pytest

from oracle import e4m3, logits, paged, schedule, topk
from tests import (test_oracle_e4m3 as pe, test_oracle_logits as pl,
                   test_oracle_schedule as ps, test_oracle_topk as pt)


def _encode_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    j = ex.astype(np.int64) - 1
    sub = a < 2.0 ** -6
    qexp = np.where(sub, -9, j - 3)
    n = np.floor(np.ldexp(a, -qexp) + 0.5)               # mistake: ties away from zero
    mag = np.minimum(np.where(sub, n, (j + 6) * 8 + n), 0x7E).astype(np.int64)
    return (mag | (neg << 7)).astype(np.uint8)


def _encode_unsigned_zero(x):
    c = e4m3.encode.__wrapped__(x) if hasattr(e4m3.encode, "__wrapped__") else _ORIG_ENCODE(x)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)   # mistake: drops -0


def _row_relu_after_weight(q8_t, w_t, cache, bt, p):
    q = e4m3.decode(q8_t).reshape(-1, 128)
    codes, ks = paged.read_tokens(cache, bt, np.arange(p + 1))
    d = q @ e4m3.decode(codes).T
    return np.maximum(np.asarray(w_t, np.float64)[:, None] * d, 0).sum(0) * ks


def _row_no_scale(q8_t, w_t, cache, bt, p):
    q = e4m3.decode(q8_t).reshape(-1, 128)
    codes, ks = paged.read_tokens(cache, bt, np.arange(p + 1))
    d = q @ e4m3.decode(codes).T
    return (np.asarray(w_t, np.float64)[:, None] * np.maximum(d, 0)).sum(0)


def _row_exclusive(q8_t, w_t, cache, bt, p):
    return _ORIG_ROW(q8_t, w_t, cache, bt, p)[:p] if p > 0 else _ORIG_ROW(q8_t, w_t, cache, bt, p)


def _select_high_index_ties(scores, k):
    s = np.asarray(scores, np.float64)
    pos = np.arange(s.shape[0])
    order = np.lexsort((-pos, -s))                       # mistake: higher position wins ties
    return np.sort(order[:min(k, s.shape[0])])


def _is_full_offset_off_by_one(layer_id, use_index_cache=False, freq=1, pattern=None, offset=2):
    if not use_index_cache:
        return True
    if pattern is None:
        return max(layer_id - offset, 0) % freq == 0     # mistake: drops the +1
    if 0 <= layer_id < len(pattern):
        return pattern[layer_id] != "S"
    return True


_ORIG_ENCODE = e4m3.encode
_ORIG_ROW = logits.logits_row

MUTANTS = [
    ("encode ties away from zero", e4m3, "encode", _encode_half_up, [pe.test_encode_midpoints_go_to_even]),
    ("encode loses negative zero", e4m3, "encode", _encode_unsigned_zero, [pe.test_encode_signed_zero_and_saturation]),
    ("ReLU after weighting", logits, "logits_row", _row_relu_after_weight, [pl.test_hand_computed_case]),
    ("K scale dropped", logits, "logits_row", _row_no_scale, [pl.test_hand_computed_case]),
    ("own position excluded", logits, "logits_row", _row_exclusive, [pl.test_causal_range_includes_self]),
    ("ties to higher position", topk, "select", _select_high_index_ties, [pt.test_select_matches_rank_counting]),
    ("schedule offset off by one", schedule, "is_full", _is_full_offset_off_by_one, [ps.test_schedule_hand_table]),
]


@pytest.mark.parametrize("name,mod,attr,mutant,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(monkeypatch, name, mod, attr, mutant, pins):
    monkeypatch.setattr(mod, attr, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()

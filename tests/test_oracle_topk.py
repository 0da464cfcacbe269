"""Pins for the oracle's top-k selection (CPU only)."""

import numpy as np

from oracle import topk


def _rank_bruteforce(scores, k):
    """Position i is selected iff fewer than k others beat it (higher score,
    or equal score at a lower position).  O(n^2) counting, no sort."""
    s = [float(v) for v in scores]
    sel = []
    for i in range(len(s)):
        better = sum(1 for j in range(len(s)) if s[j] > s[i] or (s[j] == s[i] and j < i))
        if better < k:
            sel.append(i)
    return sel


def test_select_matches_rank_counting():
    rng = np.random.default_rng(3)
    for n, k in [(1, 1), (5, 2), (40, 7), (100, 100), (100, 150), (257, 64), (300, 1)]:
        for kind in ("normal", "ties"):
            if kind == "normal":
                s = rng.standard_normal(n)
            else:
                s = rng.integers(-3, 4, n).astype(np.float64)
            got = topk.select(s, k)
            assert list(got) == _rank_bruteforce(s, k)


def test_row_layout_and_padding():
    s = np.array([0.1, 5.0, -2.0, 5.0, 3.0])
    row = topk.topk_row(s, 3)
    assert row.dtype == np.int32
    assert list(row) == [1, 3, 4]                 # ascending positions
    row = topk.topk_row(s, 8)
    assert list(row) == [0, 1, 2, 3, 4, -1, -1, -1]


def test_all_equal_takes_lowest_positions():
    s = np.full(50, 1.25)
    assert list(topk.select(s, 10)) == list(range(10))


def test_signed_zeros_are_equal():
    s = np.array([-0.0, 0.0, -0.0, 0.0, -1.0])
    assert list(topk.select(s, 2)) == [0, 1]


def test_planted_peaks_are_found():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(5000)
    hot = rng.choice(5000, 20, replace=False)
    s[hot] += 10.0
    assert set(topk.select(s, 20)) == set(hot)


def test_kth_value():
    s = np.array([1.0, 9.0, 3.0, 7.0])
    assert topk.kth_value(s, 2) == 7.0
    assert topk.kth_value(s, 10) == 1.0

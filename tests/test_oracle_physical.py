"""Pins for the oracle's logical -> physical top-k conversion (CPU only)."""

import numpy as np

from oracle import physical


def test_hand_computed_conversion():
    # two requests, block_size 4; request 0 owns blocks [7, 2], request 1 owns [5]
    block_table = np.array([[7, 2], [5, -1]])
    logical = np.array([[0, 5, -1], [3, 1, 2], [6, -1, -1]], np.int32)
    token_req = np.array([0, 1, 0])
    out, valid = physical.to_physical(logical, token_req, block_table, block_size=4)
    # pos 0 -> block 7 off 0 = 28; pos 5 -> block 2 off 1 = 9; pos 3 (req 1) -> 5*4+3 = 23
    assert out.tolist() == [[28, 9, -1], [23, 21, 22], [10, -1, -1]]
    assert valid.tolist() == [2, 3, 1]


def test_block_stride_rows():
    out, _ = physical.to_physical(np.array([[1, 4]]), np.array([0]), np.array([[3, 6]]),
                                  block_size=4, stride=10)
    assert out.tolist() == [[31, 60]]

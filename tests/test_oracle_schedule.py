"""Pins for the oracle's IndexCache schedule and stack (CPU only)."""

import json
import os

import numpy as np

from oracle import Batch, quant, schedule, stack
from synth import random_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_table.json")


def test_schedule_hand_table():
    for c in json.load(open(GOLDEN))["cases"]:
        got = schedule.schedule(c["num_layers"], c["use_index_cache"], c["freq"],
                                c["pattern"], c["offset"])
        assert "".join("F" if f else "S" for f in got) == c["expect"], c


def test_pr_report_form_equals_blog_form_at_default_offset():
    # the PR report writes the frequency rule as max(layer_id - 1, 0) % freq
    for freq in range(1, 7):
        for layer in range(40):
            pr = max(layer - 1, 0) % freq == 0
            assert schedule.is_full(layer, True, freq, None, 2) == pr


def test_pattern_errors():
    assert schedule.pattern_errors("FSSS", 4) == []
    assert "length" in schedule.pattern_errors("FSS", 4)
    assert "alphabet" in schedule.pattern_errors("FSxS", 4)
    assert "first-layer-S" in schedule.pattern_errors("SFFF", 4)


def _stack_layers(wl, num_layers):
    layers = []
    for layer in range(num_layers):
        kb, slots = wl.new_rows(layer)
        cache = np.zeros((wl.num_blocks, 64, 132), np.uint8)
        cb, cs = wl.ctx_rows(layer)
        quant.quant_write_k(cache, cb, cs)
        q8, qs = quant.quantize_q(wl.q_bits(layer))
        w = quant.fold_weights(wl.w_raw(layer), qs)
        layers.append(dict(cache=cache, k_bits=kb, slot_mapping=slots, q8=q8, w=w))
    return layers


def test_stack_s_layers_consume_last_f_rows():
    wl = random_batch(77, [150, 90, 200], [1, 1, 1], k=16, num_layers=6)
    batch = Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    full = schedule.schedule(6, True, 1, "FSSFSF", 2)
    out = stack.run_stack(_stack_layers(wl, 6), full, batch, wl.k)
    for s_layer, f_layer in [(1, 0), (2, 0), (4, 3)]:
        for t in out[f_layer]:
            assert np.array_equal(out[s_layer][t], out[f_layer][t])
    # F layers use their own q, w and K, so their rows differ from the previous F layer's
    assert any(not np.array_equal(out[3][t], out[0][t]) for t in out[0])


def test_stack_writes_k_on_every_layer():
    wl = random_batch(78, [70], [2], k=8, num_layers=2)
    batch = Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    layers = _stack_layers(wl, 2)
    before = layers[1]["cache"].copy()
    stack.run_stack(layers, [True, False], batch, wl.k)
    assert not np.array_equal(before, layers[1]["cache"])     # S layer's K written
    layers = _stack_layers(wl, 2)
    before = layers[1]["cache"].copy()
    stack.run_stack(layers, [True, False], batch, wl.k, write_k_on_s=False)
    assert np.array_equal(before, layers[1]["cache"])

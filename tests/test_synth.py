"""The seeded generators: determinism and layout validity (CPU only)."""

import numpy as np

from synth import CONFIGS, f32_to_bf16_bits, make_workload, random_batch


def test_bf16_rounding_known_values():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -8 + 2 ** -20], np.float32)
    # ties go to even: 1 + 2^-8 is halfway between 0x3F80 and 0x3F81 -> 0x3F80
    assert f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_workloads_are_deterministic_and_valid():
    for name, spec in CONFIGS.items():
        a, b = make_workload(spec), make_workload(spec)
        assert np.array_equal(a.seq_lens, b.seq_lens)
        assert np.array_equal(a.block_table, b.block_table)
        assert np.all(a.seq_lens >= spec.len_lo) and np.all(a.seq_lens <= spec.len_hi)
        used = np.concatenate([a.block_table[r, :-(-int(L) // 64)] for r, L in enumerate(a.seq_lens)])
        assert np.unique(used).size == used.size                    # no shared physical block
        assert used.min() >= 0 and used.max() < a.num_blocks
        assert a.num_tokens == spec.num_reqs * spec.new_tokens


def test_draws_repeat_per_request():
    wl = random_batch(5, [100, 300], [2, 1], k=8, planted=3)
    assert np.array_equal(wl.request_k(0, 1), wl.request_k(0, 1))
    assert not np.array_equal(wl.request_k(0, 1)[:100], wl.request_k(1, 1)[:100])
    kb, slots = wl.new_rows(0)
    assert kb.shape == (3, 128) and slots.shape == (3,)
    assert np.array_equal(kb[2], wl.request_k(0, 1)[299])
    cb, cs = wl.ctx_rows(0)
    assert cb.shape == (98 + 299, 128)
    assert np.unique(np.concatenate([cs, slots])).size == 400
    assert wl.token_pos().tolist() == [98, 99, 299]

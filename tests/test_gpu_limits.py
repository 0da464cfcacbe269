"""GPU parity at the size limits of the top-k, for empty batches, and for
rows whose scores are all equal.

Long rows are filtered in chunks (2048 positions on the fused path, which has
the scoring kernel's sample copy; 4096 for idx_topk alone), one candidate slot
per chunk.  Rows of up to 128 slots have their candidates preloaded by the
resolve work-group while the slot counts are still in flight; longer rows are
gathered after the counts.  The rows here reach the library's longest row,
2^22 positions.
"""

import numpy as np
import pytest

import oracle
from oracle import topk as otopk
from synth import random_batch
from tests.gpu_helpers import (check_topk_band, device_batch, device_layer, oracle_batch,
                               oracle_layer, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_fp8_amd as m
    return m, torch


def test_topk_longest_rows(env):
    """idx_topk alone: 300 000 positions (74 slots, preloaded), 600 000 (147
    slots) and 2^22 - 5 (1024 slots, the longest row accepted), exact against
    the oracle's full sort."""
    m, torch = env
    lengths = [300_000, 600_000, (1 << 22) - 5]
    k = 2048
    wl = random_batch(3101, lengths, 1, k=k)
    rng = np.random.default_rng(3101)
    scores = np.full((wl.num_tokens, wl.max_seq_len), np.nan, np.float32)
    for t, n in enumerate(wl.seq_lens):
        scores[t, :n] = rng.standard_normal(int(n)).astype(np.float32)
    say("longest rows", lengths)
    got = m.idx_topk(torch.from_numpy(scores).cuda(), device_batch(m, wl), k).cpu().numpy()
    for t, n in enumerate(wl.seq_lens):
        want = otopk.topk_row(scores[t, :n].astype(np.float64), k)
        assert np.array_equal(got[t], want), f"row {t} n={n}"


@pytest.mark.parametrize("lengths", [[300_000], [300_000, 70_000]])
def test_score_topk_long_row_past_preload(env, lengths):
    """The fused path on one request of 300 000 positions alone (chunks of 19
    blocks: 247 slots, more than the resolve preloads, gathered after the
    counts) and beside one of 70 000 (127 and 30 slots of 37 blocks): equal to
    idx_logits + idx_topk and within the oracle's tie band."""
    m, torch = env
    wl = random_batch(3102, lengths, 1, k=2048)
    say("fused long rows", wl.seq_lens.tolist())
    dev = device_layer(m, torch, wl, 0, with_new=True)
    batch = device_batch(m, wl)
    lg = m.idx_logits(dev["q8"], dev["w"], dev["cache"], batch)
    a = m.idx_topk(lg, batch, wl.k).cpu().numpy()
    b = m.idx_score_topk(dev["q8"], dev["w"], dev["cache"], batch, wl.k).cpu().numpy()
    assert np.array_equal(a, b)
    orc = oracle_layer(wl, 0)
    ob = oracle_batch(wl)
    for t in range(wl.num_tokens):
        r, p = ob.token_request(t), ob.token_position(t)
        want = oracle.logits.logits_row(orc["q8"][t], orc["w"][t], orc["cache"], wl.block_table[r], p)
        check_topk_band(b[t], want, wl.k, f"token {t}")


def test_empty_batch(env):
    """A batch with no new tokens launches nothing and returns empty results."""
    m, torch = env
    batch = m.Batch([5, 9], [0, 0, 0], [[0], [1]])
    cache = m.KCache(2, fill=0)
    q8 = torch.empty((0, 64, 128), dtype=torch.uint8, device="cuda")
    w = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    assert m.idx_logits(q8, w, cache, batch).shape[0] == 0
    assert m.idx_score_topk(q8, w, cache, batch, 16).shape == (0, 16)
    lg = torch.empty((0, 9), dtype=torch.float32, device="cuda")
    assert m.idx_topk(lg, batch, 16).shape == (0, 16)
    torch.cuda.synchronize()


def test_score_topk_all_scores_equal(env):
    """Head weights all zero (and, separately, q all zero) make every score
    exactly +0: each row then selects its lowest k positions, on the few-long-
    rows shape (every position a candidate, more than the LDS list holds) and
    on the many-rows shape, fused and unfused alike."""
    m, torch = env
    for wl in (random_batch(3103, [100, 3000, 20000, 70000], 1, k=2048),
               random_batch(3104, [5000, 300], [200, 60], k=256)):
        dev = device_layer(m, torch, wl, 0, with_new=True)
        batch = device_batch(m, wl)
        for what, q8, w in (("w = 0", dev["q8"], torch.zeros_like(dev["w"])),
                            ("q = 0", torch.zeros_like(dev["q8"]), dev["w"])):
            lg = m.idx_logits(q8, w, dev["cache"], batch)
            a = m.idx_topk(lg, batch, wl.k).cpu().numpy()
            b = m.idx_score_topk(q8, w, dev["cache"], batch, wl.k).cpu().numpy()
            lg = lg.cpu().numpy()
            ob = oracle_batch(wl)
            for t in range(wl.num_tokens):
                n = ob.token_position(t) + 1
                assert np.all(lg[t, :n].view(np.uint32) == 0), f"{what} token {t}: scores not +0"
                want = np.full(wl.k, -1, np.int32)
                want[:min(n, wl.k)] = np.arange(min(n, wl.k))
                assert np.array_equal(a[t], want), f"{what} token {t} (unfused)"
                assert np.array_equal(b[t], want), f"{what} token {t} (fused)"

"""idx_score_topk_noalloc (the entry point that allocates nothing: its
workspace is the library's per-device array) against idx_score_topk with a
caller workspace, through the C ABI.

Two calls in a row, the second on a smaller batch, so the second runs on an
array that still holds the first call's contents.  Top-k rows are integers:
the two entry points must agree element by element.
"""

import numpy as np
import pytest

from synth import random_batch
from tests.gpu_helpers import check_topk_band, device_batch, device_layer, oracle_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_fp8_amd as m
    return m, torch


def _one(m, torch, wl, what):
    say(f"[noalloc] {what}: lengths {wl.seq_lens.tolist()} new {wl.new_tokens.tolist()} k {wl.k}")
    dev = device_layer(m, torch, wl, 0, with_new=True)
    batch = device_batch(m, wl)
    need = m.idx_score_topk_workspace_size(batch, wl.k)
    assert 0 < need <= m.binding.NOALLOC_SCRATCH_BYTES, need
    want = m.idx_score_topk(dev["q8"], dev["w"], dev["cache"], batch, wl.k)
    got = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    m.idx_score_topk_noalloc(dev["q8"], dev["w"], dev["cache"], batch, wl.k, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{what}: rows differ from idx_score_topk"
    return dev, got.cpu().numpy()


def test_noalloc_two_calls_second_smaller(env):
    m, torch = env
    import oracle
    # long decode rows (the filter + resolve shape), then a smaller prefill batch
    big = random_batch(7101, [20000, 9000, 14000, 4100], 1, k=2048)
    small = random_batch(7102, [700, 1500], [64, 9], k=256)
    for wl, what in ((big, "first call"), (small, "second call, smaller")):
        dev, got = _one(m, torch, wl, what)
        # and the rows are the oracle's (tie band of the k-th score)
        orc = oracle_layer(wl, 0)
        ob = oracle.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
        for t in range(0, wl.num_tokens, max(1, wl.num_tokens // 8)):
            r, p = ob.token_request(t), ob.token_position(t)
            s = oracle.logits.logits_row(orc["q8"][t], orc["w"][t], orc["cache"], wl.block_table[r], p)
            check_topk_band(got[t], s, wl.k, f"{what} token {t}")


def test_noalloc_rejects_batches_beyond_the_array(env):
    m, torch = env
    # 2048 prefill tokens over 32K positions: the scores alone need 256 MiB
    wl = random_batch(7103, [32768], [2048], k=2048)
    batch = device_batch(m, wl)
    assert m.idx_score_topk_workspace_size(batch, wl.k) > m.binding.NOALLOC_SCRATCH_BYTES
    q8 = torch.zeros((wl.num_tokens, 64, 128), dtype=torch.uint8, device="cuda")
    w = torch.zeros((wl.num_tokens, 64), dtype=torch.float32, device="cuda")
    cache = m.KCache(wl.num_blocks, fill=0)
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(m.IdxError) as e:
        m.idx_score_topk_noalloc(q8, w, cache, batch, wl.k, topk)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((topk == -7).all()), "a rejected call launched something"

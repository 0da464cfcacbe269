"""GPU parity at the five workloads' full sizes, on sampled rows.

The GPU runs each whole configuration exactly as the bench times it (new K
rows written, then the fused score + top-k); the oracle recomputes a sample
of query tokens one by one from the same raw draws.
"""

import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_workload
from tests.gpu_helpers import (check_logits_row, check_topk_band, device_batch, device_layer,
                               oracle_batch, oracle_layer, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_fp8_amd as m
    return m, torch


def _sample_tokens(wl, count):
    T = wl.num_tokens
    if T <= count:
        return list(range(T))
    return sorted(set(np.linspace(0, T - 1, count).astype(int).tolist()))


def _check_config(m, torch, name, n_sample):
    wl = make_workload(CONFIGS[name])
    say(f"[{name}] tokens {wl.num_tokens} max_seq_len {wl.max_seq_len} pool {wl.num_blocks}")
    dev = device_layer(m, torch, wl, 0)
    batch = device_batch(m, wl)
    # the timed step: write this step's K rows, then score + select
    m.idx_quant_write_k(dev["k_new"], dev["slots_new"], dev["cache"])
    topk = m.idx_score_topk(dev["q8"], dev["w"], dev["cache"], batch, wl.k)
    logits = m.idx_logits(dev["q8"], dev["w"], dev["cache"], batch)
    torch.cuda.synchronize()
    got_topk = topk.cpu().numpy()
    tokens = _sample_tokens(wl, n_sample)
    reqs = sorted(set(int(r) for r in wl.token_req()[tokens]))
    say(f"[{name}] oracle on tokens {tokens} (requests {reqs})")
    orc = oracle_layer(wl, 0, reqs=reqs)
    ob = oracle_batch(wl)
    for t in tokens:
        r = ob.token_request(t)
        p = ob.token_position(t)
        # the oracle cache holds only the sampled requests: compare their bytes too
        blocks = wl.block_table[r, : (p + 64) // 64]
        assert np.array_equal(dev["cache"].tensor[torch.from_numpy(blocks.astype(np.int64)).cuda()].cpu().numpy(),
                              orc["cache"][blocks]), f"token {t}: cache bytes"
        want = oracle.logits.logits_row(orc["q8"][t], orc["w"][t], orc["cache"], wl.block_table[r], p)
        check_logits_row(logits[t, : p + 1].cpu().numpy(), want, f"{name} token {t}")
        check_topk_band(got_topk[t], want, wl.k, f"{name} token {t}")
    return wl, orc, got_topk


def test_prefill_1k(env):
    m, torch = env
    _check_config(m, torch, "prefill-1k", 64)


def test_decode_64x16k_32k(env):
    m, torch = env
    _check_config(m, torch, "decode-64x16k-32k", 5)


def test_prefill_24k_8k(env):
    m, torch = env
    _check_config(m, torch, "prefill-24k+8k", 6)


def test_decode_8x128k_planted(env):
    m, torch = env
    wl, orc, got = _check_config(m, torch, "decode-8x128k", 2)
    # planted rows (K x3) score three times further from zero; with signed head
    # weights about a quarter of them land far in the positive tail, so they are
    # selected far more often than the base rate k / n
    base = wl.k / wl.max_seq_len
    fracs = []
    for t in range(wl.num_tokens):
        hot = wl.planted_positions(t)
        fracs.append(np.isin(hot, got[t]).mean())
        say(f"token {t}: planted selected {fracs[-1]:.2f} (base rate {base:.3f})")
        assert fracs[-1] > base, f"token {t}"
    assert np.mean(fracs) > 5 * base


def test_stack_16L_32x64k(env):
    m, torch = env
    wl = make_workload(CONFIGS["stack-16L-32x64k"])
    full = m.idx_layer_schedule(True, wl.pattern, 1, 2, wl.num_layers)
    assert full == [c == "F" for c in wl.pattern]
    batch = device_batch(m, wl)
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(batch, wl.k), dtype=torch.uint8, device="cuda")
    consumed = []
    sample_reqs = [0, 31]
    f_rows = {}
    for layer in range(wl.num_layers):
        say(f"[stack] layer {layer} {'F' if full[layer] else 'S'}")
        dev = device_layer(m, torch, wl, layer)
        m.idx_indexcache_layer(dev["k_new"], dev["cache"], dev["q8"], dev["w"], full[layer], True,
                               dev["slots_new"], batch, wl.k, topk, workspace=ws)
        torch.cuda.synchronize()
        consumed.append(topk.cpu().numpy().copy())
        # the new K rows were written on every layer, S layers included
        r = 5
        p = int(wl.seq_lens[r]) - 1
        blk = int(wl.block_table[r, p // 64])
        cb = dev["cache"].tensor[blk].cpu().numpy().reshape(-1)
        assert not np.all(cb[(p % 64) * 128:(p % 64) * 128 + 128] == 0xEE), f"layer {layer}: K not written"
        if full[layer]:
            orc = oracle_layer(wl, layer, reqs=sample_reqs)
            for t in sample_reqs:
                want = oracle.logits.logits_row(orc["q8"][t], orc["w"][t], orc["cache"],
                                                 wl.block_table[t], int(wl.seq_lens[t]) - 1)
                check_topk_band(consumed[-1][t], want, wl.k, f"layer {layer} token {t}")
            f_rows[layer] = consumed[-1]
        del dev
    last_f = None
    for layer in range(wl.num_layers):
        if full[layer]:
            last_f = layer
        else:
            assert np.array_equal(consumed[layer], consumed[last_f]), f"S layer {layer}"
    assert not np.array_equal(consumed[0], consumed[4])

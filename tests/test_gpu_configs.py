"""GPU parity at the five workloads' full sizes, on the step the bench times.

Each test builds the device state the way bench.py does (the cached context K
written with idx_quant_write_k, q quantised and the weights folded with
idx_quant_q_fold_w), runs one F layer exactly as the bench times it
(idx_indexcache_layer with is_full = 1 and write_k = 1; on decode batches the
scoring kernel itself writes the step's new K rows) and compares with the
oracle, recomputed on the host from the same raw draws:

  * the whole K cache, byte for byte, new rows included;
  * the top-k row of every query token (130 stratified tokens of the
    8192-token prefill chunk) against the oracle's fp64 scores, with the tie
    band of the k-th score.

The 16-layer stack also compares the new K rows of every layer, S layers
included, with oracle bytes, checks every row of each F layer against the
oracle, checks that S layers leave the last F layer's rows in the buffer,
and runs each layer with the group's physical conversion: after an F layer
the physical rows and valid counts equal the oracle's conversion of its
top-k rows, and an S layer leaves them as they were.
"""

import numpy as np
import pytest

from oracle import quant as oquant
from oracle.physical import to_physical
from synth import CONFIGS, make_workload
from tests.gpu_helpers import (check_topk_band, device_batch, device_layer, oracle_layer,
                               oracle_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_fp8_amd as m
    return m, torch


def _timed_step(m, torch, wl, dev, batch):
    """One F layer as bench.py times it: new K rows, scores, top-k."""
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(batch, wl.k), dtype=torch.uint8, device="cuda")
    m.idx_indexcache_layer(dev["k_new"], dev["cache"], dev["q8"], dev["w"], True, True,
                           dev["slots_new"], batch, wl.k, topk, workspace=ws)
    torch.cuda.synchronize()
    return topk.cpu().numpy()


def _check_config(m, torch, name, tokens=None):
    wl = make_workload(CONFIGS[name])
    say(f"[{name}] tokens {wl.num_tokens} max_seq_len {wl.max_seq_len} pool {wl.num_blocks}")
    dev = device_layer(m, torch, wl, 0)
    batch = device_batch(m, wl)
    got = _timed_step(m, torch, wl, dev, batch)
    say(f"[{name}] oracle cache for {wl.num_reqs} requests")
    orc = oracle_layer(wl, 0)
    assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"]), "K cache bytes"
    tokens = range(wl.num_tokens) if tokens is None else tokens
    tokens = sorted(set(int(t) for t in tokens))
    say(f"[{name}] oracle scores for {len(tokens)} query tokens")
    want = oracle_rows(wl, orc, tokens)
    for t in tokens:
        check_topk_band(got[t], want[t], wl.k, f"{name} token {t}")
    return wl, got


def test_prefill_1k(env):
    m, torch = env
    _check_config(m, torch, "prefill-1k")


def test_decode_64x16k_32k(env):
    m, torch = env
    _check_config(m, torch, "decode-64x16k-32k")


def test_prefill_24k_8k(env):
    """130 of the 8192 tokens: every offset within a group of 8 (the prefill
    kernel's tokens per work-group) in 16 groups spread over the chunk, and
    both ends of the range."""
    m, torch = env
    groups = np.linspace(0, 8192 // 8 - 1, 16).astype(int)
    tokens = [g * 8 + o for g in groups for o in range(8)] + [0, 8191]
    _check_config(m, torch, "prefill-24k+8k", tokens)


def test_decode_8x128k_planted(env):
    m, torch = env
    wl, got = _check_config(m, torch, "decode-8x128k")
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


def _new_row_bytes(cache_tensor, slots):
    """[n, 132] bytes (128 codes, 4 scale bytes) of the given slots of a device cache."""
    flat = cache_tensor.view(cache_tensor.shape[0], -1).cpu().numpy()
    out = np.zeros((len(slots), 132), np.uint8)
    for i, s in enumerate(slots):
        b, off = divmod(int(s), 64)
        out[i, :128] = flat[b, off * 128:(off + 1) * 128]
        out[i, 128:] = flat[b, 64 * 128 + off * 4:64 * 128 + off * 4 + 4]
    return out


def test_stack_16L_32x64k(env):
    m, torch = env
    wl = make_workload(CONFIGS["stack-16L-32x64k"])
    full = m.idx_layer_schedule(True, wl.pattern, 1, 2, wl.num_layers)
    assert full == [c == "F" for c in wl.pattern]
    batch = device_batch(m, wl)
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(batch, wl.k), dtype=torch.uint8, device="cuda")
    # the group's physical rows: converted after each F layer, left alone by S layers
    phys = m.Physical(wl.num_tokens, wl.k, wl.num_blocks, fill=-9)
    consumed = []
    for layer in range(wl.num_layers):
        say(f"[stack] layer {layer} {'F' if full[layer] else 'S'}")
        dev = device_layer(m, torch, wl, layer)
        before = (phys.physical.cpu().numpy().copy(), phys.valid_counts.cpu().numpy().copy())
        m.idx_indexcache_layer_physical(dev["k_new"], dev["cache"], dev["q8"], dev["w"], full[layer],
                                        True, dev["slots_new"], batch, wl.k, topk, phys,
                                        workspace=ws)
        torch.cuda.synchronize()
        consumed.append(topk.cpu().numpy().copy())
        got_phys = (phys.physical.cpu().numpy(), phys.valid_counts.cpu().numpy())
        if full[layer]:
            want_phys = to_physical(consumed[-1], wl.token_req(), wl.block_table, 64)
        else:
            want_phys = before
        assert np.array_equal(got_phys[0], want_phys[0]), f"layer {layer}: physical rows"
        assert np.array_equal(got_phys[1], want_phys[1]), f"layer {layer}: valid counts"
        # this layer's new K rows (written inside scoring on F layers, by the
        # separate quantiser on S layers) against the oracle's bytes
        nb, ns = wl.new_rows(layer)
        codes, scales = oquant.quantize_rows(nb)
        want = np.concatenate([codes, scales.astype("<f4").view(np.uint8).reshape(-1, 4)], axis=1)
        assert np.array_equal(_new_row_bytes(dev["cache"].tensor, ns), want), f"layer {layer}: K rows"
        if full[layer]:
            orc = oracle_layer(wl, layer)
            assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"]), \
                f"layer {layer}: K cache bytes"
            scores = oracle_rows(wl, orc, range(wl.num_tokens))
            for t in range(wl.num_tokens):
                check_topk_band(consumed[-1][t], scores[t], wl.k, f"layer {layer} token {t}")
            del orc, scores
        del dev
    last_f = None
    for layer in range(wl.num_layers):
        if full[layer]:
            last_f = layer
        else:
            assert np.array_equal(consumed[layer], consumed[last_f]), f"S layer {layer}"
    assert not np.array_equal(consumed[0], consumed[4])

"""GPU parity of the FP4 indexer K cache against the oracle (oracle.fp4cache).

Cache bytes must be identical (every finite bf16 value included); scores
within the scoring tolerance of the oracle's fp64 scores on the same decoded
K; the decode and prefill scoring kernels give the same bits; top-k rows
equal idx_topk over idx_logits_fp4 and fall inside the oracle's tie band.
The full-size case runs the FP4 step of 8 decode tokens over 128K positions
(idx_indexcache_layer_fp4: the fused scoring kernel writes the new K rows,
keeps its scores on chip and passes per-chunk candidates to the exact
select) and checks the whole cache and every row.
"""

import numpy as np
import pytest

import oracle
from oracle import fp4cache
from synth import CONFIGS, f32_to_bf16_bits, make_workload, random_batch
from tests.fp8_bruteforce import all_finite_bf16_bits
from tests.gpu_helpers import (adversarial_q_w, check_logits_row, check_topk_band, device_batch,
                               device_layer, oracle_batch, oracle_layer, oracle_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_fp8_amd as m
    return m, torch


def _special_rows(rng):
    """Rows whose groups hit the quantiser's edge cases."""
    x = rng.standard_normal((48, 4, 32)) * np.ldexp(1.0, rng.integers(-10, 10, (48, 4, 1)))
    x[0] = 0.0                                   # all zero: floor exponent in every group
    x[1, 1] = -0.0
    x[2, 2] = 1e-6                               # below the amax floor
    x[3, :, :] = 0.0
    x[3, 0, 7] = 6.0 * 2 ** 5                    # amax exactly on a boundary
    x[3, 1, 9] = -6.0 * 2 ** -3
    x[4] *= 1e30                                 # near the top of the bf16 range
    x[5] *= 1e-30                                # bf16 subnormals
    x[6, 3, ::2] = 0.25 * 2 ** 2                 # exact ties (0.25, 1.25, 2.5, 5 times 2^e) ...
    x[6, 3, 1::2] = 5.0 * 2 ** 2                 # ... with amax 5*4 -> e = 2
    x[7, 0] = np.linspace(-6, 6, 32) * 2 ** -1
    return f32_to_bf16_bits(x.reshape(48, 128).astype(np.float32))


# ------------------------------------------------------------ quantiser --

def test_fp4_quant_write_k_bitexact(env):
    m, torch = env
    rng = np.random.default_rng(7101)
    bits = np.concatenate([_special_rows(rng),
                           f32_to_bf16_bits(rng.standard_normal((1000, 128)).astype(np.float32))])
    nb = 20
    slots = rng.permutation(nb * 64)[:bits.shape[0]].astype(np.int64)
    slots[::17] = -1                             # padding tokens
    slots[5] = nb * 64 + 3                       # outside the pool: skipped
    say("fp4 quant_write_k: rows", bits.shape[0], "pool", nb)
    cache = m.KCacheFP4(nb, fill=0xA5)
    m.idx_quant_write_k_fp4(torch.from_numpy(bits.view(np.int16)).cuda(),
                            torch.from_numpy(slots).cuda(), cache)
    want = fp4cache.new_cache(nb, fill=0xA5)
    keep = slots < nb * 64
    fp4cache.quant_write_k(want, bits[keep], slots[keep])
    assert np.array_equal(cache.tensor.cpu().numpy(), want)


def test_fp4_quant_strided_rows(env):
    m, torch = env
    rng = np.random.default_rng(7102)
    full = f32_to_bf16_bits(rng.standard_normal((300, 192)).astype(np.float32))
    slots = np.arange(300, dtype=np.int64)
    cache = m.KCacheFP4(5, fill=0)
    t = torch.from_numpy(full.view(np.int16)).cuda()
    m.idx_quant_write_k_fp4(t[:, :128], torch.from_numpy(slots).cuda(), cache)
    want = fp4cache.new_cache(5)
    fp4cache.quant_write_k(want, np.ascontiguousarray(full[:, :128]), slots)
    assert np.array_equal(cache.tensor.cpu().numpy(), want)


def test_fp4_quant_all_finite_bf16_patterns(env):
    """Every finite bf16 value, in groups of similar magnitude (sorted) and of
    mixed magnitude (shuffled)."""
    m, torch = env
    bits = all_finite_bf16_bits()
    bits = np.concatenate([bits, np.zeros((-bits.size) % 128, np.uint16)])
    rng = np.random.default_rng(7103)
    for arrangement in ("sorted", "shuffled"):
        rows = (bits if arrangement == "sorted" else rng.permutation(bits)).reshape(-1, 128)
        nb = -(-rows.shape[0] // 64)
        slots = np.arange(rows.shape[0], dtype=np.int64)
        cache = m.KCacheFP4(nb, fill=0)
        m.idx_quant_write_k_fp4(torch.from_numpy(rows.view(np.int16)).cuda(),
                                torch.from_numpy(slots).cuda(), cache)
        want = fp4cache.new_cache(nb)
        fp4cache.quant_write_k(want, rows, slots)
        got = cache.tensor.cpu().numpy()
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{arrangement}: {bad.shape[0]} bytes differ, first {bad[:3].tolist()}"


# --------------------------------------------------------------- scores --

def _run_logits(m, torch, wl, note, num_decode_tokens=0):
    dev = device_layer(m, torch, wl, 0, with_new=True, fmt="fp4")
    orc = oracle_layer(wl, 0, fmt="fp4")
    assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"]), note
    batch = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table,
                    num_decode_tokens=num_decode_tokens)
    logits = torch.full((wl.num_tokens, wl.max_seq_len + 5), float("nan"), device="cuda")
    m.idx_logits_fp4(dev["q8"], dev["w"], dev["cache"], batch, logits=logits)
    got = logits.cpu().numpy()
    want = oracle_rows(wl, orc, range(wl.num_tokens))
    for t, row in want.items():
        n = row.shape[0]
        check_logits_row(got[t, :n], row, f"{note} token {t}")
        assert np.all(np.isnan(got[t, n:])), f"{note} token {t}: wrote past p_t"
    return dev, orc, got


def test_fp4_logits_decode_ragged(env):
    m, torch = env
    wl = random_batch(7201, [1, 63, 64, 65, 127, 1000, 3000, 4097], 1, k=64)
    say("fp4 logits decode ragged", wl.seq_lens.tolist())
    _run_logits(m, torch, wl, "fp4 decode")


def test_fp4_logits_prefill_ragged(env):
    m, torch = env
    wl = random_batch(7202, [100, 1500, 64, 700], [100, 37, 10, 1], k=64)
    say("fp4 logits prefill ragged", wl.seq_lens.tolist(), wl.new_tokens.tolist())
    _run_logits(m, torch, wl, "fp4 prefill")


def test_fp4_decode_and_prefill_kernels_agree_bitwise(env):
    """Requests of three new tokens scored with the decode split
    (num_decode_tokens = all) and with the prefill split: the same bits."""
    m, torch = env
    wl = random_batch(7203, [2000, 700, 5000, 130], 3, k=64)
    say("fp4 decode vs prefill split", wl.seq_lens.tolist())
    dev, orc, pre = _run_logits(m, torch, wl, "fp4 prefill split")
    dec = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table, num_decode_tokens=wl.num_tokens)
    got = m.idx_logits_fp4(dev["q8"], dev["w"], dev["cache"], dec).cpu().numpy()
    pos = wl.token_pos()
    for t in range(wl.num_tokens):
        n = int(pos[t]) + 1
        assert np.array_equal(got[t, :n].view(np.uint32), pre[t, :n].view(np.uint32)), t


def test_fp4_logits_linear_half_adversarial(env):
    m, torch = env
    L, T = 3000, 12
    wl = random_batch(7204, [L], T, k=64)
    dev = device_layer(m, torch, wl, 0, with_new=True, fmt="fp4")
    orc = oracle_layer(wl, 0, fmt="fp4")
    assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"])
    q8, w = adversarial_q_w(np.random.default_rng(7204), T)
    got = m.idx_logits_fp4(torch.from_numpy(q8).cuda(), torch.from_numpy(w).cuda(), dev["cache"],
                           device_batch(m, wl)).cpu().numpy()
    want = fp4cache.logits(q8, w, orc["cache"], oracle_batch(wl))
    for t, row in want.items():
        check_logits_row(got[t, :row.shape[0]], row, f"fp4 adversarial token {t}")
    assert np.all(got[4, :L - T + 5].view(np.uint32) == 0)


@pytest.mark.parametrize("new", [1, 37])
def test_fp4_logits_absent_blocks(env, new):
    """Block-table entries of -1 or outside the pool: the call completes and the
    other positions' scores equal the oracle's."""
    m, torch = env
    wl = random_batch(7205, [4000, 2500], new, k=64)
    dev = device_layer(m, torch, wl, 0, with_new=True, fmt="fp4")
    orc = oracle_layer(wl, 0, fmt="fp4")
    bt = wl.block_table.copy()
    absent = {(0, 3): -1, (0, 40): wl.num_blocks, (1, 0): -7, (1, 20): wl.num_blocks + 100}
    for (r, lb), v in absent.items():
        bt[r, lb] = v
    batch = m.Batch(wl.seq_lens, wl.query_start_loc, bt)
    got = m.idx_logits_fp4(dev["q8"], dev["w"], dev["cache"], batch).cpu().numpy()
    want = oracle_rows(wl, orc, range(wl.num_tokens))
    for t, row in want.items():
        r = int(np.searchsorted(wl.query_start_loc, t, side="right") - 1)
        keep = np.ones(row.shape[0], bool)
        for (rr, lb), _ in absent.items():
            if rr == r:
                keep[lb * 64:(lb + 1) * 64] = False
        check_logits_row(got[t, :row.shape[0]][keep], row[keep], f"fp4 absent blocks, token {t}")


# ---------------------------------------------------------------- top-k --

@pytest.mark.parametrize("lengths,new,k", [
    ([20000, 9000, 30000, 1500], 1, 2048),        # decode rows long enough for the long-row select
    ([3000, 700], [200, 40], 256),                # prefill chunks
])
def test_fp4_score_topk(env, lengths, new, k):
    m, torch = env
    wl = random_batch(7301 + len(lengths), lengths, new, k=k)
    say("fp4 score_topk", lengths, new, k)
    dev = device_layer(m, torch, wl, 0, with_new=True, fmt="fp4")
    batch = device_batch(m, wl)
    got = m.idx_score_topk_fp4(dev["q8"], dev["w"], dev["cache"], batch, k)
    lg = m.idx_logits_fp4(dev["q8"], dev["w"], dev["cache"], batch)
    assert np.array_equal(got.cpu().numpy(), m.idx_topk(lg, batch, k).cpu().numpy())
    orc = oracle_layer(wl, 0, fmt="fp4")
    assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"])
    want = oracle_rows(wl, orc, range(wl.num_tokens))
    g = got.cpu().numpy()
    for t in range(wl.num_tokens):
        check_topk_band(g[t], want[t], k, f"fp4 token {t}")


def _fp4_scale_positions(dev_cache, orc_cache, block_table_row, positions, add):
    """Add `add` to the four E8M0 group exponents of the given logical positions in
    both FP4 caches: their scores scale by exactly 2^add."""
    import torch
    p = np.asarray(positions, np.int64)
    b = np.asarray(block_table_row, np.int64)[p // 64].repeat(4)
    q = (p % 64).repeat(4)
    g = np.tile(np.arange(4), p.size)
    off = 4096 + g * 64 + (q % 16) * 4 + q // 16
    orc_cache[b, off] = (orc_cache[b, off].astype(np.int64) + add).astype(np.uint8)
    dev_cache.tensor[torch.from_numpy(b).cuda(), torch.from_numpy(off).cuda()] = \
        torch.from_numpy(orc_cache[b, off].copy()).cuda()


def test_fp4_fused_rescore_fallback(env):
    """Decode rows over long contexts take the fused path over the FP4 cache
    too.  2048 consecutive positions of request 0 scaled by 8 (their group
    exponents + 3) hold far more than their chunks' share of the top k, so the
    row is rescored whole; the rows equal idx_logits_fp4 + idx_topk and the
    oracle's band."""
    m, torch = env
    wl = random_batch(7401, [20000, 9000, 30000], 1, k=2048)
    dev = device_layer(m, torch, wl, 0, with_new=True, fmt="fp4")
    orc = oracle_layer(wl, 0, fmt="fp4")
    hot = list(range(8192, 8192 + 2048))
    _fp4_scale_positions(dev["cache"], orc["cache"], wl.block_table[0], hot, 3)
    assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"])
    batch = device_batch(m, wl)
    lg = m.idx_logits_fp4(dev["q8"], dev["w"], dev["cache"], batch)
    a = m.idx_topk(lg, batch, wl.k).cpu().numpy()
    with m.KernelTrace(capacity=8) as tr:
        b = m.idx_score_topk_fp4(dev["q8"], dev["w"], dev["cache"], batch, wl.k)
    assert [n for n, _ in tr.kernels] == ["score_keep_fp4_kernel", "topk_keep_resolve_kernel"]
    b = b.cpu().numpy()
    assert np.array_equal(a, b)
    want = oracle_rows(wl, orc, range(wl.num_tokens))
    for t in range(wl.num_tokens):
        check_topk_band(b[t], want[t], wl.k, f"fp4 fallback token {t}")
    assert np.isin(hot, b[0]).sum() > 700, "the scaled positions should dominate row 0"


def test_fp4_layer_k_write_inside_scoring(env):
    """idx_indexcache_layer_fp4 on an F layer: the cache bytes and the top-k rows
    equal the separate idx_quant_write_k_fp4 + idx_logits_fp4 + idx_topk on a
    copy of the cache: decode batches over long rows (the fused kernel writes
    the new rows itself) with a padding token, requests of three new tokens
    with the decode split (fused, rows written inside scoring) and without it
    (prefill split, rows written first), and many short requests (unfused)."""
    m, torch = env
    many = np.random.default_rng(7403).integers(1, 6000, 40).tolist()
    cases = [(random_batch(7401, [3000, 9000, 20000, 700, 1500], 1, k=512), [0], [3]),
             (random_batch(7402, [2500, 9000, 4000], 3, k=256), [9, 0], []),
             (random_batch(7403, many, 1, k=256), [0], [5])]
    for wl, splits, pad in cases:
        for nd in splits:
            say("fp4 layer K write", wl.seq_lens.tolist(), wl.new_tokens.tolist(), "decode tokens", nd)
            dev = device_layer(m, torch, wl, 0, fmt="fp4")
            slots = dev["slots_new"].clone()
            for p in pad:
                slots[p] = -1
            batch = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table, num_decode_tokens=nd)
            ref_cache = m.KCacheFP4(wl.num_blocks, tensor=dev["cache"].tensor.clone())
            m.idx_quant_write_k_fp4(dev["k_new"], slots, ref_cache)
            lg = m.idx_logits_fp4(dev["q8"], dev["w"], ref_cache, batch)
            want = m.idx_topk(lg, batch, wl.k).cpu().numpy()
            topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
            m.idx_indexcache_layer_fp4(dev["k_new"], dev["cache"], dev["q8"], dev["w"], True, True,
                                       slots, batch, wl.k, topk)
            assert torch.equal(dev["cache"].tensor, ref_cache.tensor)
            assert np.array_equal(topk.cpu().numpy(), want)
    # an S layer writes the rows and nothing else
    wl = random_batch(7404, [3000, 9000], 1, k=256)
    dev = device_layer(m, torch, wl, 0, fmt="fp4")
    batch = device_batch(m, wl)
    ref_cache = m.KCacheFP4(wl.num_blocks, tensor=dev["cache"].tensor.clone())
    m.idx_quant_write_k_fp4(dev["k_new"], dev["slots_new"], ref_cache)
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    m.idx_indexcache_layer_fp4(dev["k_new"], dev["cache"], dev["q8"], dev["w"], False, True,
                               dev["slots_new"], batch, wl.k, topk)
    assert torch.equal(dev["cache"].tensor, ref_cache.tensor)
    assert bool((topk == -7).all())


def test_fp4_candidate_stages(env):
    """idx_score_candidates_fp4 + idx_select_candidates_fp4 are the FP4 fused
    path's two launches: the same cache bytes and rows as the F layer."""
    m, torch = env
    wl = random_batch(7405, [20000, 9000, 30000], 1, k=2048)
    dev = device_layer(m, torch, wl, 0, fmt="fp4")
    batch = device_batch(m, wl)
    ref_cache = m.KCacheFP4(wl.num_blocks, tensor=dev["cache"].tensor.clone())
    ref = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    m.idx_indexcache_layer_fp4(dev["k_new"], ref_cache, dev["q8"], dev["w"], True, True,
                               dev["slots_new"], batch, wl.k, ref)
    ws = torch.empty(m.idx_score_topk_fp4_workspace_size(batch, wl.k), dtype=torch.uint8,
                     device="cuda")
    m.idx_score_candidates_fp4(dev["q8"], dev["w"], dev["cache"], batch, wl.k, ws, dev["k_new"],
                               dev["slots_new"])
    got = m.idx_select_candidates_fp4(dev["q8"], dev["w"], dev["cache"], batch, wl.k, ws)
    assert torch.equal(dev["cache"].tensor, ref_cache.tensor)
    assert torch.equal(got, ref)


def test_fp4_decode_8x128k_step(env):
    """The FP4 step at full size, as bench.py times it: 8 decode tokens over
    128K positions through idx_indexcache_layer_fp4.  The whole cache against
    the oracle's bytes, every row against its fp64 scores."""
    m, torch = env
    wl = make_workload(CONFIGS["decode-8x128k"])
    say(f"[fp4 decode-8x128k] tokens {wl.num_tokens} pool {wl.num_blocks}")
    dev = device_layer(m, torch, wl, 0, fmt="fp4")
    batch = device_batch(m, wl)
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_fp4_workspace_size(batch, wl.k), dtype=torch.uint8,
                     device="cuda")
    m.idx_indexcache_layer_fp4(dev["k_new"], dev["cache"], dev["q8"], dev["w"], True, True,
                               dev["slots_new"], batch, wl.k, topk, workspace=ws)
    torch.cuda.synchronize()
    say("[fp4 decode-8x128k] oracle cache")
    orc = oracle_layer(wl, 0, fmt="fp4")
    assert np.array_equal(dev["cache"].tensor.cpu().numpy(), orc["cache"]), "FP4 cache bytes"
    say("[fp4 decode-8x128k] oracle scores")
    want = oracle_rows(wl, orc, range(wl.num_tokens))
    got = topk.cpu().numpy()
    for t in range(wl.num_tokens):
        check_topk_band(got[t], want[t], wl.k, f"fp4 decode-8x128k token {t}")

"""Shared setup for the GPU parity tests.

Both sides start from the same raw draws of ``synth``: the HIP library
quantises and scatters K and quantises q / folds w with its own kernels, the
oracle does the same on the CPU; tests then compare.
"""

import concurrent.futures as cf
import os
import sys

import numpy as np

import oracle
from oracle import quant as oquant

TOL_ABS = 1e-3
TOL_REL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ----------------------------------------------------------------- device --

def device_batch(m, wl):
    return m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)


def device_ctx_rows(wl, layer):
    """All cached-context K rows of one layer, drawn request by request in parallel."""
    reqs = [r for r in range(wl.num_reqs) if wl.seq_lens[r] > wl.new_tokens[r]]
    if not reqs:
        return np.zeros((0, 128), np.uint16), np.zeros(0, np.int64)

    def one(r):
        return wl.ctx_rows(layer, [r])

    with cf.ThreadPoolExecutor(workers()) as ex:
        parts = list(ex.map(one, reqs))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def device_layer(m, torch, wl, layer, fill=0xEE, with_new=False, fmt="fp8"):
    """A device cache holding the layer's context K (written by idx_quant_write_k,
    or idx_quant_write_k_fp4 for an FP4 cache), plus the layer's q_fp8 / folded
    w (from idx_quant_q_fold_w) and new K rows."""
    fp4 = fmt == "fp4"
    cache = (m.KCacheFP4 if fp4 else m.KCache)(wl.num_blocks, fill=fill)
    write = m.idx_quant_write_k_fp4 if fp4 else m.idx_quant_write_k
    kb, slots = device_ctx_rows(wl, layer)
    if kb.shape[0]:
        kt = torch.from_numpy(kb.view(np.int16)).cuda()
        st = torch.from_numpy(slots).cuda()
        write(kt, st, cache)
        del kt, st
    qb = torch.from_numpy(wl.q_bits(layer).view(np.int16)).cuda()
    wr = torch.from_numpy(wl.w_raw(layer)).cuda()
    q8, w, qs = m.idx_quant_q_fold_w(qb, wr)
    nb, ns = wl.new_rows(layer)
    out = dict(cache=cache, q8=q8, w=w, qs=qs,
               k_new=torch.from_numpy(nb.view(np.int16)).cuda(),
               slots_new=torch.from_numpy(ns).cuda())
    if with_new:
        write(out["k_new"], out["slots_new"], cache)
    return out


# ----------------------------------------------------------------- oracle --

def oracle_batch(wl):
    return oracle.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)


def oracle_layer(wl, layer, reqs=None, with_new=True, fill=0xEE, fmt="fp8"):
    """The oracle's cache (only the requests in ``reqs``; FP8, or FP4 with
    fmt="fp4") and q8 / folded w.  Requests own disjoint blocks, so they are
    quantised and written in parallel threads (numpy releases the GIL in the
    heavy steps)."""
    reqs = list(range(wl.num_reqs) if reqs is None else reqs)
    if fmt == "fp4":
        cache = oracle.fp4cache.new_cache(wl.num_blocks, fill)
        write = oracle.fp4cache.quant_write_k
    else:
        cache = np.full((wl.num_blocks, 64, 132), fill, np.uint8)
        write = oquant.quant_write_k

    def one(r):
        kb = wl.request_k(layer, r)
        L, n = int(wl.seq_lens[r]), int(wl.new_tokens[r])
        upto = L if with_new else L - n
        write(cache, kb[:upto], wl.slots(r, np.arange(upto)))

    with cf.ThreadPoolExecutor(workers()) as ex:
        list(ex.map(one, reqs))
    q8, qs = oquant.quantize_q(wl.q_bits(layer))
    w = oquant.fold_weights(wl.w_raw(layer), qs)
    return dict(cache=cache, q8=q8, qs=qs, w=w, fmt=fmt)


def oracle_rows(wl, orc, tokens):
    """Oracle scores {t: fp64 row} for the given query tokens, in parallel
    threads (one BLAS thread each)."""
    ob = oracle_batch(wl)
    row = oracle.fp4cache.logits_row if orc.get("fmt") == "fp4" else oracle.logits.logits_row

    def one(t):
        r, p = ob.token_request(int(t)), ob.token_position(int(t))
        return int(t), row(orc["q8"][t], orc["w"][t], orc["cache"], wl.block_table[r], p)

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:                              # pragma: no cover - optional
        limit = None
    try:
        with cf.ThreadPoolExecutor(workers()) as ex:
            return dict(ex.map(one, tokens))
    finally:
        if limit is not None:
            limit.restore_original_limits()


# ------------------------------------------------------------- inputs --

def adversarial_q_w(rng, T):
    """q codes and folded weights chosen to stress the scores' linear half.

    The scoring kernels split w*max(d, 0) into (w/2)|d| + (w/2)d and contract
    the second half as u . k with u = sum_h (w_h/2) q_h held in four E4M3
    pieces; these rows give u a wide dynamic range, saturated codes, exact
    cancellation and weights over several decades.
    """
    H, D = 64, 128
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    q8 = rng.choice(finite, size=(T, H, D)).astype(np.uint8)
    # four decades of weights, up to ~10x the folded weights of N(0,1) data (larger ones make
    # the plain fp32 head sum itself miss the tolerance where the terms cancel)
    w = (rng.choice([-1.0, 1.0], size=(T, H)) * 10.0 ** rng.uniform(-7, -3, size=(T, H))).astype(np.float32)
    q8[0] = 0x7E                                  # every code +448: u is w-weighted sum of 448s
    q8[1, :, :] = 0x01                            # smallest subnormal everywhere ...
    q8[1, :, 0] = 0x7E                            # ... but one dimension at +448: u spans ~2^18
    w[2, 1::2] = -w[2, 0::2]                      # pairs of heads with opposite weights ...
    q8[2, 1::2] = q8[2, 0::2]                     # ... and equal q rows: every score is 0 (u = 0)
    q8[3] = np.where(rng.random((H, D)) < 0.5, 0x80, q8[3])   # half the codes -0
    w[4] = 0.0                                    # all weights zero
    w[5] = np.float32(1e-30)                      # tiny weights (u far below the clamp range)
    return q8, w


# ------------------------------------------------------------- comparison --

def check_logits_row(got, want, what=""):
    """|g - o| <= 1e-3 + 1e-3 |o| on the causal range."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    bound = TOL_ABS + TOL_REL * np.abs(want)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, (f"{what}: {bad.size} logits out of tolerance, first at {bad[:5]}, "
                           f"got {got[bad[:5]]}, want {want[bad[:5]]}")


def check_topk_band(row, scores, k, what=""):
    """GPU top-k row against oracle fp64 scores with the tie band of the k-th score."""
    row = np.asarray(row)
    n = scores.shape[0]
    nsel = min(k, n)
    sel = row[:nsel]
    assert np.all(row[nsel:] == -1), f"{what}: padding"
    assert np.all((sel >= 0) & (sel < n)), f"{what}: positions outside 0..p_t"
    assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
    if n <= k:
        assert np.array_equal(sel, np.arange(n)), f"{what}: short row must take every position"
        return
    vk = oracle.topk.kth_value(scores, k)
    tau = TOL_ABS + TOL_REL * abs(vk)
    chosen = np.zeros(n, bool)
    chosen[sel] = True
    must = scores > vk + tau
    never = scores < vk - tau
    assert np.all(chosen[must]), f"{what}: missed {np.count_nonzero(must & ~chosen)} clear winners"
    assert not np.any(chosen[never]), f"{what}: took {np.count_nonzero(never & chosen)} clear losers"

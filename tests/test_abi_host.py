"""The C ABI on the host: exported symbols and argument checks (no GPU calls).

Every call below is rejected by host-side validation before any launch, so
fake device addresses are safe: the library never dereferences them on the host.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")
LIB = os.path.join(ROOT, "sparse_attention_token_fp8_amd", "libidx.so")


@pytest.fixture(scope="module")
def m():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._builder().build()
    import sparse_attention_token_fp8_amd as pkg
    return pkg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(m):
    names = declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(m.binding.SIGNATURES), "binding misses a declared entry point"


def _batch(m, num_reqs=1, num_tokens=1, max_seq_len=64, max_query_len=1, stride=1, null=False,
           num_decode_tokens=0):
    fake = 0 if null else 0x10000
    return m.binding.BatchC(fake, fake, fake, stride, num_reqs, num_tokens, max_seq_len, max_query_len,
                            num_decode_tokens)


FAKE = ctypes.c_void_p(0x10000)
S = ctypes.c_void_p(0)


def _cache(m, nb=4, bs=64, data=0x10000):
    return m.binding.KCacheC(data, nb, bs)


def test_quant_write_k_rejects(m):
    L = m.lib()
    assert L.idx_quant_write_k(FAKE, 1, 64, 128, FAKE, _cache(m), S) == -2          # head_dim
    assert L.idx_quant_write_k(FAKE, 1, 128, 128, FAKE, _cache(m, bs=16), S) == -2  # block_size
    assert L.idx_quant_write_k(FAKE, -1, 128, 128, FAKE, _cache(m), S) == -1
    assert L.idx_quant_write_k(None, 1, 128, 128, FAKE, _cache(m), S) == -1
    assert L.idx_quant_write_k(FAKE, 1, 128, 126, FAKE, _cache(m), S) == -1         # stride % 4
    assert L.idx_quant_write_k(FAKE, 1, 128, 64, FAKE, _cache(m), S) == -1          # stride < 128
    assert L.idx_quant_write_k(ctypes.c_void_p(0x10002), 1, 128, 128, FAKE, _cache(m), S) == -1
    assert L.idx_quant_write_k(FAKE, 1, 128, 128, FAKE, _cache(m, data=0x10004), S) == -1
    assert L.idx_quant_write_k(FAKE, 1, 128, 128, ctypes.c_void_p(0x10004), _cache(m), S) == -1  # slots
    assert L.idx_quant_write_k(FAKE, 0, 128, 128, FAKE, _cache(m), S) == 0           # no-op


def test_scoring_rejects(m):
    L = m.lib()
    B = ctypes.byref
    ok = _batch(m)
    assert L.idx_logits(FAKE, FAKE, 32, 128, _cache(m), B(ok), FAKE, 64, S) == -2
    assert L.idx_logits(FAKE, FAKE, 64, 64, _cache(m), B(ok), FAKE, 64, S) == -2
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), None, FAKE, 64, S) == -1
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, null=True)), FAKE, 64, S) == -1
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, num_reqs=0)), FAKE, 64, S) == -1
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(ok), FAKE, 63, S) == -1    # ld < max_seq_len
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, max_seq_len=65)), FAKE, 65, S) == -1
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, num_tokens=70000)), FAKE, 64, S) == -2
    assert L.idx_logits(ctypes.c_void_p(0x10008), FAKE, 64, 128, _cache(m), B(ok), FAKE, 64, S) == -1
    odd = ctypes.c_void_p(0x10002)
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(ok), odd, 64, S) == -1     # logits
    bad = m.binding.BatchC(0x10002, 0x10000, 0x10000, 1, 1, 1, 64, 1, 0)             # seq_lens
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(bad), FAKE, 64, S) == -1
    for nd in (-1, 2):                                          # decode split outside 0..num_tokens
        assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, num_decode_tokens=nd)),
                            FAKE, 64, S) == -1
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, num_tokens=0, max_query_len=0)),
                        None, 64, S) == 0


def test_topk_rejects(m):
    L = m.lib()
    B = ctypes.byref
    ok = _batch(m, num_tokens=4, max_query_len=4)
    need = L.idx_topk_workspace_size(B(ok), 16)
    assert need > 0
    assert L.idx_topk(FAKE, 64, B(ok), 0, FAKE, 16, FAKE, need, S) == -2
    assert L.idx_topk(FAKE, 64, B(ok), 4096, FAKE, 4096, FAKE, 1 << 30, S) == -2
    assert L.idx_topk(FAKE, 64, B(ok), 16, FAKE, 8, FAKE, need, S) == -1             # stride < k
    assert L.idx_topk(FAKE, 64, B(ok), 16, ctypes.c_void_p(0x10002), 16, FAKE, need, S) == -1  # topk
    assert L.idx_topk(FAKE, 64, B(ok), 16, FAKE, 16, FAKE, need - 1, S) == -3
    assert L.idx_topk(FAKE, 64, B(ok), 16, FAKE, 16, None, need, S) == -3
    assert L.idx_topk(FAKE, 64, B(ok), 16, FAKE, 16, ctypes.c_void_p(0x10010), need, S) == -3
    sneed = L.idx_score_topk_workspace_size(B(ok), 16)
    assert sneed > need                                         # the fused path also holds scores
    assert L.idx_score_topk(FAKE, FAKE, 64, 128, _cache(m), B(ok), 16, FAKE, 16, FAKE, sneed - 1, S) == -3


def test_schedule_matches_oracle_and_rejects(m):
    from oracle import schedule as osched
    for freq in (1, 2, 3, 4):
        for off in (1, 2, 3):
            want = osched.schedule(12, True, freq, None, off)
            if not want[0]:
                with pytest.raises(m.IdxError):
                    m.idx_layer_schedule(True, None, freq, off, 12)
                continue
            assert m.idx_layer_schedule(True, None, freq, off, 12) == want
    assert m.idx_layer_schedule(True, "FSSS" * 4, 1, 2, 16) == osched.schedule(16, True, 1, "FSSS" * 4, 2)
    assert m.idx_layer_schedule(False, None, 4, 2, 5) == [True] * 5
    for bad in [("FSS", 4), ("FSxS", 4), ("SFFF", 4), ("", 1)]:
        with pytest.raises(m.IdxError):
            m.idx_layer_schedule(True, bad[0], 1, 2, bad[1])
    with pytest.raises(m.IdxError):
        m.idx_layer_schedule(True, None, 0, 2, 4)


def test_stack_rejects_s_first_and_bad_layers(m):
    L = m.lib()
    B = ctypes.byref
    io = (m.binding.LayerIOC * 2)()
    full = (ctypes.c_uint8 * 2)(0, 1)
    ok = _batch(m)
    assert L.idx_indexcache_stack(io, 2, ctypes.cast(full, ctypes.c_void_p), 1, FAKE, B(ok), 8,
                                  FAKE, 8, FAKE, 1 << 20, S) == -1
    full = (ctypes.c_uint8 * 2)(1, 0)
    io[0].cache = _cache(m)
    io[0].k_bf16, io[0].k_row_stride, io[0].q_fp8, io[0].w = 0x10000, 128, 0x10000, 0x10000
    io[1].cache = _cache(m, bs=32)
    assert L.idx_indexcache_stack(io, 2, ctypes.cast(full, ctypes.c_void_p), 1, FAKE, B(ok), 8,
                                  FAKE, 8, FAKE, 1 << 20, S) == -2


def test_physical_rejects(m):
    L = m.lib()
    B = ctypes.byref
    ok = _batch(m)
    assert L.idx_topk_to_physical(FAKE, 8, B(ok), 64, 10, 0, 0, FAKE, 8, None, S) == -2
    assert L.idx_topk_to_physical(FAKE, 8, B(ok), 0, 10, 8, 0, FAKE, 8, None, S) == -1
    assert L.idx_topk_to_physical(FAKE, 8, B(ok), 64, 10, 8, 32, FAKE, 8, None, S) == -1  # stride < bs
    assert L.idx_topk_to_physical(FAKE, 8, B(ok), 64, 1 << 30, 8, 64, FAKE, 8, None, S) == -2


def test_quant_q_fold_requires_16_byte_q_fp8(m):
    L = m.lib()
    # q_fp8 only 4-byte aligned: rejected before any launch (the 16-lane kernel stores 8 bytes)
    assert L.idx_quant_q_fold_w(FAKE, FAKE, 1, 64, 128, 0.088, ctypes.c_void_p(0x10004), FAKE,
                                None, S) == -1
    assert L.idx_quant_q_fold_w(FAKE, FAKE, 1, 64, 128, 0.088, ctypes.c_void_p(0x10008), FAKE,
                                None, S) == -1


def test_physical_checks_table_width_against_its_block_size(m):
    L = m.lib()
    B = ctypes.byref
    # 1024 positions in blocks of 128 need 8 table entries: accepted up to the pointer checks
    # (a null physical pointer then gives -1 only after the batch passed)
    wide = _batch(m, max_seq_len=1024, stride=8)
    assert L.idx_topk_to_physical(FAKE, 8, B(wide), 128, 10, 8, 0, None, 8, None, S) == -1
    assert L.idx_topk_to_physical(FAKE, 8, B(_batch(m, max_seq_len=1024, stride=8, num_tokens=0,
                                                    max_query_len=0)),
                                  128, 10, 8, 0, FAKE, 8, None, S) == 0
    # seven entries are too few for 1024 positions in blocks of 128
    narrow = _batch(m, max_seq_len=1024, stride=7, num_tokens=0, max_query_len=0)
    assert L.idx_topk_to_physical(FAKE, 8, B(narrow), 128, 10, 8, 0, FAKE, 8, None, S) == -1
    # the scoring calls still need one entry per 64 positions
    assert L.idx_logits(FAKE, FAKE, 64, 128, _cache(m), B(_batch(m, max_seq_len=1024, stride=8,
                                                                 num_tokens=0, max_query_len=0)),
                        FAKE, 1024, S) == -1


def test_trace_rejects_and_ends_empty(m):
    L = m.lib()
    assert L.idx_trace_begin(None, 8) == -1
    assert L.idx_trace_begin(FAKE, 1) == -1
    assert L.idx_trace_end(None, 0) == 0              # not tracing: nothing bracketed
    # tracing, but every call below is rejected on the host: no kernel, no event recorded
    assert L.idx_trace_begin(FAKE, 8) == 0
    assert L.idx_quant_write_k(FAKE, 1, 64, 128, FAKE, _cache(m), S) == -2
    assert L.idx_trace_end(None, 0) == 0


def test_candidate_stages_reject_other_batches(m):
    L = m.lib()
    B = ctypes.byref
    # a prefill batch (4 new tokens of one request): not the fused path
    pre = _batch(m, num_tokens=4, max_seq_len=20000, max_query_len=4, stride=400)
    assert L.idx_score_candidates(FAKE, FAKE, 64, 128, _cache(m), B(pre), 2048, None, 0, None,
                                  FAKE, 1 << 30, S) == -2
    assert L.idx_select_candidates(FAKE, FAKE, 64, 128, _cache(m), B(pre), 2048, FAKE, 2048,
                                   FAKE, 1 << 30, S) == -2
    # a decode batch over long rows is the fused path: a short workspace is refused
    dec = _batch(m, num_tokens=1, max_seq_len=20000, max_query_len=1, stride=400)
    need = L.idx_score_topk_workspace_size(B(dec), 2048)
    assert need > 0
    assert L.idx_score_candidates(FAKE, FAKE, 64, 128, _cache(m), B(dec), 2048, None, 0, None,
                                  FAKE, need - 1, S) == -3
    assert L.idx_select_candidates(FAKE, FAKE, 64, 128, _cache(m), B(dec), 2048, FAKE, 2048,
                                   FAKE, need - 1, S) == -3
    assert L.idx_score_candidates(FAKE, FAKE, 64, 128, _cache(m), B(dec), 0, None, 0, None,
                                  FAKE, need, S) == -2


def test_group_physical_rejects_before_any_work(m):
    L = m.lib()
    B = ctypes.byref
    ok = _batch(m)
    io = (m.binding.LayerIOC * 2)()
    for lay in io:
        lay.cache = _cache(m)
        lay.k_bf16, lay.k_row_stride, lay.q_fp8, lay.w = 0x10000, 128, 0x10000, 0x10000
    full = ctypes.cast((ctypes.c_uint8 * 2)(1, 0), ctypes.c_void_p)
    P = m.binding.PhysicalC
    bad = [P(0x10000, 8, None, 0, 10, 0),            # block size 0
           P(0x10000, 4, None, 64, 10, 0),           # physical rows narrower than k
           P(0x10000, 8, None, 64, 10, 32),          # block stride below the block size
           P(None, 8, None, 64, 10, 0),              # no physical rows for a non-empty batch
           P(0x10002, 8, None, 64, 10, 0)]           # misaligned rows
    want = [-1, -1, -1, -1, -1]
    for ph, w in zip(bad, want):
        # an F layer checks the physical arguments before it scores anything
        assert L.idx_indexcache_layer_physical(B(io[0]), 1, 1, FAKE, B(ok), 8, FAKE, 8, B(ph),
                                               FAKE, 1 << 20, S) == w
        assert L.idx_indexcache_stack_physical(io, 2, full, 1, FAKE, B(ok), 8, FAKE, 8, B(ph),
                                               FAKE, 1 << 20, S) == w
    huge = P(0x10000, 8, None, 64, 1 << 30, 64)          # pool beyond int32 slots
    assert L.idx_indexcache_stack_physical(io, 2, full, 1, FAKE, B(ok), 8, FAKE, 8, B(huge),
                                           FAKE, 1 << 20, S) == -2
    # a good physical description does not let a bad stack through
    good = P(0x10000, 8, None, 64, 10, 0)
    io[1].cache = _cache(m, bs=32)
    assert L.idx_indexcache_stack_physical(io, 2, full, 1, FAKE, B(ok), 8, FAKE, 8, B(good),
                                           FAKE, 1 << 20, S) == -2


@pytest.mark.parametrize("tokens,max_len", [(8, 131072), (64, 32768), (32, 65536), (1, 300000),
                                             (2, 9000), (255, 8193)])
def test_fused_workspace_follows_the_chunking(m, tokens, max_len):
    """Decode batches over long rows (fewer than 256 tokens, rows past 8192
    positions) take the fused path, whose workspace holds per (row, chunk) a
    candidate slot of chunk-size (key, position) pairs and three words of
    summary.  Chunks cover about one CU's share of the batch's blocks, 8 to
    128 blocks of 64 positions; the FP4 cache uses the same layout."""
    L = m.lib()
    B = ctypes.byref
    bpr = -(-max_len // 64)
    cb = min(128, max(8, -(-bpr * tokens // 256)))
    cap = cb * 64
    nslots = -(-max_len // cap)
    up = lambda x: -(-x // 256) * 256
    want = up(8 * tokens * nslots * cap) + 3 * up(4 * tokens * nslots)
    dec = _batch(m, num_reqs=tokens, num_tokens=tokens, max_seq_len=max_len, max_query_len=1,
                 stride=bpr)
    assert L.idx_score_topk_workspace_size(B(dec), 2048) == want
    assert L.idx_score_topk_fp4_workspace_size(B(dec), 2048) == want

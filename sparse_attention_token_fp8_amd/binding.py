"""ctypes binding of libidx.  Argument marshalling only: every step runs in
the library's HIP kernels; torch supplies device memory and the stream.

The functions carry the C names (``idx_quant_write_k`` ...) and take torch
tensors.  A status other than IDX_OK raises ``IdxError``.  Importing this
module fails loudly if libidx.so has not been built.
"""

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidx.so")

N_HEADS = 64
HEAD_DIM = 128
BLOCK_SIZE = 64
TOKEN_BYTES = 132

IDX_OK = 0
STATUS_NAMES = {0: "IDX_OK", -1: "IDX_ERR_INVALID_ARG", -2: "IDX_ERR_UNSUPPORTED",
                -3: "IDX_ERR_WORKSPACE", -4: "IDX_ERR_LAUNCH"}


class IdxError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({_lib.idx_status_str(status).decode()})")


class KCacheC(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32)]


class BatchC(ctypes.Structure):
    _fields_ = [("seq_lens", ctypes.c_void_p), ("query_start_loc", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
                ("num_reqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("max_query_len", ctypes.c_int32),
                ("num_decode_tokens", ctypes.c_int32)]


class LayerIOC(ctypes.Structure):
    _fields_ = [("k_bf16", ctypes.c_void_p), ("k_row_stride", ctypes.c_int64),
                ("cache", KCacheC), ("q_fp8", ctypes.c_void_p), ("w", ctypes.c_void_p)]


class PhysicalC(ctypes.Structure):
    _fields_ = [("physical", ctypes.c_void_p), ("physical_stride", ctypes.c_int64),
                ("valid_counts", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("block_stride_rows", ctypes.c_int64)]


_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_PBatch = ctypes.POINTER(BatchC)

SIGNATURES = {
    "idx_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "idx_version": (ctypes.c_char_p, []),
    "idx_quant_write_k": (ctypes.c_int, [_vp, _i64, _i32, _i64, _vp, KCacheC, _vp]),
    "idx_quant_q_fold_w": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp]),
    "idx_logits": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _vp, _i64, _vp]),
    "idx_topk_workspace_size": (_sz, [_PBatch, _i32]),
    "idx_topk": (ctypes.c_int, [_vp, _i64, _PBatch, _i32, _vp, _i64, _vp, _sz, _vp]),
    "idx_score_topk_workspace_size": (_sz, [_PBatch, _i32]),
    "idx_score_topk": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp, _i64,
                                      _vp, _sz, _vp]),
    "idx_score_topk_noalloc": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp,
                                              _i64, _vp]),
    "idx_score_candidates": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp, _i64,
                                            _vp, _vp, _sz, _vp]),
    "idx_select_candidates": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp,
                                             _i64, _vp, _sz, _vp]),
    "idx_quant_write_k_fp4": (ctypes.c_int, [_vp, _i64, _i32, _i64, _vp, KCacheC, _vp]),
    "idx_logits_fp4": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _vp, _i64, _vp]),
    "idx_score_topk_fp4_workspace_size": (_sz, [_PBatch, _i32]),
    "idx_score_topk_fp4": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp, _i64,
                                          _vp, _sz, _vp]),
    "idx_score_candidates_fp4": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp,
                                                _i64, _vp, _vp, _sz, _vp]),
    "idx_select_candidates_fp4": (ctypes.c_int, [_vp, _vp, _i32, _i32, KCacheC, _PBatch, _i32, _vp,
                                                 _i64, _vp, _sz, _vp]),
    "idx_indexcache_layer_fp4": (ctypes.c_int, [ctypes.POINTER(LayerIOC), _i32, _i32, _vp, _PBatch,
                                                _i32, _vp, _i64, _vp, _sz, _vp]),
    "idx_layer_schedule": (ctypes.c_int, [_i32, ctypes.c_char_p, _i32, _i32, _i32, _vp]),
    "idx_trace_begin": (ctypes.c_int, [_vp, _i32]),
    "idx_trace_end": (_i32, [_vp, _i32]),
    "idx_indexcache_layer": (ctypes.c_int, [ctypes.POINTER(LayerIOC), _i32, _i32, _vp, _PBatch,
                                            _i32, _vp, _i64, _vp, _sz, _vp]),
    "idx_indexcache_stack": (ctypes.c_int, [ctypes.POINTER(LayerIOC), _i32, _vp, _i32, _vp,
                                            _PBatch, _i32, _vp, _i64, _vp, _sz, _vp]),
    "idx_indexcache_layer_physical": (ctypes.c_int, [ctypes.POINTER(LayerIOC), _i32, _i32, _vp,
                                                     _PBatch, _i32, _vp, _i64,
                                                     ctypes.POINTER(PhysicalC), _vp, _sz, _vp]),
    "idx_indexcache_stack_physical": (ctypes.c_int, [ctypes.POINTER(LayerIOC), _i32, _vp, _i32,
                                                     _vp, _PBatch, _i32, _vp, _i64,
                                                     ctypes.POINTER(PhysicalC), _vp, _sz, _vp]),
    "idx_topk_to_physical": (ctypes.c_int, [_vp, _i64, _PBatch, _i32, _i64, _i32, _i64, _vp, _i64,
                                            _vp, _vp]),
}


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python sparse_attention_token_fp8_amd/build.py` (there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def _check(fn, status):
    if status != IDX_OK:
        raise IdxError(fn, status)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ data --

class KCache:
    """A paged indexer K cache: uint8 [num_blocks, 64, 132] on the device."""

    def __init__(self, num_blocks, device="cuda", fill=None, tensor=None):
        if tensor is None:
            if fill is None:
                tensor = torch.empty((num_blocks, BLOCK_SIZE, TOKEN_BYTES), dtype=torch.uint8, device=device)
            else:
                tensor = torch.full((num_blocks, BLOCK_SIZE, TOKEN_BYTES), fill, dtype=torch.uint8, device=device)
        self.tensor = tensor
        self.num_blocks = int(tensor.shape[0])

    def c(self):
        return KCacheC(self.tensor.data_ptr(), self.num_blocks, BLOCK_SIZE)


FP4_BLOCK_BYTES = 4352        # 64 positions x (64 code bytes + 4 scale bytes)


class KCacheFP4:
    """A paged FP4 indexer K cache: uint8 [num_blocks, 4352] on the device."""

    def __init__(self, num_blocks, device="cuda", fill=None, tensor=None):
        if tensor is None:
            shape = (num_blocks, FP4_BLOCK_BYTES)
            tensor = (torch.empty(shape, dtype=torch.uint8, device=device) if fill is None
                      else torch.full(shape, fill, dtype=torch.uint8, device=device))
        self.tensor = tensor
        self.num_blocks = int(tensor.shape[0])

    def c(self):
        return KCacheC(self.tensor.data_ptr(), self.num_blocks, BLOCK_SIZE)


class Batch:
    """Device batch metadata plus the host copies the library sizes grids with."""

    def __init__(self, seq_lens, query_start_loc, block_table, device="cuda", num_decode_tokens=0):
        sl = np.asarray(seq_lens, dtype=np.int32)
        qsl = np.asarray(query_start_loc, dtype=np.int32)
        bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
        self.seq_lens = torch.from_numpy(sl).to(device)
        self.query_start_loc = torch.from_numpy(qsl).to(device)
        self.block_table = torch.from_numpy(bt).to(device)
        self.num_reqs = int(sl.shape[0])
        self.num_tokens = int(qsl[-1])
        self.max_seq_len = int(sl.max()) if sl.size else 0
        self.max_query_len = int(np.diff(qsl).max()) if sl.size else 0
        self.block_table_stride = int(bt.shape[1])
        self.num_decode_tokens = int(num_decode_tokens)
        self._c = BatchC(self.seq_lens.data_ptr(), self.query_start_loc.data_ptr(),
                         self.block_table.data_ptr(), self.block_table_stride, self.num_reqs,
                         self.num_tokens, self.max_seq_len, self.max_query_len,
                         self.num_decode_tokens)

    def c(self):
        return ctypes.byref(self._c)


def as_bf16_bits(t):
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError("expected bf16 (or its 16-bit patterns)")


# ------------------------------------------------------------- entries --

def idx_version():
    return _lib.idx_version().decode()


def idx_quant_write_k(k, slot_mapping, cache, stream=None):
    """Quantise K rows [N, >=128] (bf16) and scatter them to their slots."""
    k = as_bf16_bits(k)
    n = int(k.shape[0])
    _check("idx_quant_write_k",
           _lib.idx_quant_write_k(_ptr(k), n, HEAD_DIM, int(k.stride(0)) if n else HEAD_DIM,
                                  _ptr(slot_mapping), cache.c(), _stream(stream)))


def idx_quant_q_fold_w(q, w_raw, softmax_scale=None, q_fp8=None, w_folded=None, q_scale=None,
                       stream=None):
    """q [T, 64, 128] bf16, w_raw [T, 64] fp32 -> (q_fp8 uint8, folded w fp32, q_scale fp32)."""
    q = as_bf16_bits(q)
    T = int(q.shape[0])
    if softmax_scale is None:
        softmax_scale = float(np.float32(HEAD_DIM ** -0.5))
    dev = q.device
    q_fp8 = torch.empty((T, N_HEADS, HEAD_DIM), dtype=torch.uint8, device=dev) if q_fp8 is None else q_fp8
    w_folded = torch.empty((T, N_HEADS), dtype=torch.float32, device=dev) if w_folded is None else w_folded
    q_scale = torch.empty((T, N_HEADS), dtype=torch.float32, device=dev) if q_scale is None else q_scale
    _check("idx_quant_q_fold_w",
           _lib.idx_quant_q_fold_w(_ptr(q), _ptr(w_raw), T, N_HEADS, HEAD_DIM, softmax_scale,
                                   _ptr(q_fp8), _ptr(w_folded), _ptr(q_scale), _stream(stream)))
    return q_fp8, w_folded, q_scale


def idx_logits(q_fp8, w, cache, batch, logits=None, stream=None):
    """Scores [T, >=max_seq_len] fp32; entries past each token's position are left as they were."""
    if logits is None:
        logits = torch.empty((batch.num_tokens, max(batch.max_seq_len, 1)), dtype=torch.float32,
                             device=q_fp8.device)
    _check("idx_logits",
           _lib.idx_logits(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(),
                           _ptr(logits), int(logits.stride(0)), _stream(stream)))
    return logits


def idx_topk_workspace_size(batch, k):
    return int(_lib.idx_topk_workspace_size(batch.c(), k))


def idx_score_topk_workspace_size(batch, k):
    return int(_lib.idx_score_topk_workspace_size(batch.c(), k))


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def idx_topk(logits, batch, k, topk=None, workspace=None, stream=None):
    """[T, k] int32: selected positions ascending, then -1."""
    if topk is None:
        topk = torch.empty((batch.num_tokens, k), dtype=torch.int32, device=logits.device)
    ws = _workspace(idx_topk_workspace_size(batch, k), logits.device, workspace)
    _check("idx_topk",
           _lib.idx_topk(_ptr(logits), int(logits.stride(0)), batch.c(), k, _ptr(topk),
                         int(topk.stride(0)), _ptr(ws), ws.numel(), _stream(stream)))
    return topk


def idx_score_topk(q_fp8, w, cache, batch, k, topk=None, workspace=None, stream=None):
    if topk is None:
        topk = torch.empty((batch.num_tokens, k), dtype=torch.int32, device=q_fp8.device)
    ws = _workspace(idx_score_topk_workspace_size(batch, k), q_fp8.device, workspace)
    _check("idx_score_topk",
           _lib.idx_score_topk(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(), k,
                               _ptr(topk), int(topk.stride(0)), _ptr(ws), ws.numel(),
                               _stream(stream)))
    return topk


def idx_quant_write_k_fp4(k, slot_mapping, cache, stream=None):
    """Quantise K rows [N, >=128] (bf16) to the FP4 cache (a KCacheFP4)."""
    k = as_bf16_bits(k)
    n = int(k.shape[0])
    _check("idx_quant_write_k_fp4",
           _lib.idx_quant_write_k_fp4(_ptr(k), n, HEAD_DIM, int(k.stride(0)) if n else HEAD_DIM,
                                      _ptr(slot_mapping), cache.c(), _stream(stream)))


def idx_logits_fp4(q_fp8, w, cache, batch, logits=None, stream=None):
    """Scores against an FP4 cache, as idx_logits."""
    if logits is None:
        logits = torch.empty((batch.num_tokens, max(batch.max_seq_len, 1)), dtype=torch.float32,
                             device=q_fp8.device)
    _check("idx_logits_fp4",
           _lib.idx_logits_fp4(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(),
                               _ptr(logits), int(logits.stride(0)), _stream(stream)))
    return logits


def idx_score_topk_fp4_workspace_size(batch, k):
    return int(_lib.idx_score_topk_fp4_workspace_size(batch.c(), k))


def idx_score_topk_fp4(q_fp8, w, cache, batch, k, topk=None, workspace=None, stream=None):
    if topk is None:
        topk = torch.empty((batch.num_tokens, k), dtype=torch.int32, device=q_fp8.device)
    ws = _workspace(idx_score_topk_fp4_workspace_size(batch, k), q_fp8.device, workspace)
    _check("idx_score_topk_fp4",
           _lib.idx_score_topk_fp4(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(), k,
                                   _ptr(topk), int(topk.stride(0)), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return topk


def _score_candidates(name, q_fp8, w, cache, batch, k, workspace, k_new, slot_mapping, stream):
    kn = None if k_new is None else as_bf16_bits(k_new)
    _check(name, getattr(_lib, name)(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(),
                                     k, _ptr(kn), int(kn.stride(0)) if kn is not None else 0,
                                     _ptr(slot_mapping), _ptr(workspace), workspace.numel(),
                                     _stream(stream)))


def _select_candidates(name, q_fp8, w, cache, batch, k, workspace, topk, stream):
    if topk is None:
        topk = torch.empty((batch.num_tokens, k), dtype=torch.int32, device=q_fp8.device)
    _check(name, getattr(_lib, name)(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(),
                                     k, _ptr(topk), int(topk.stride(0)), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))
    return topk


def idx_score_candidates(q_fp8, w, cache, batch, k, workspace, k_new=None, slot_mapping=None,
                         stream=None):
    """First launch of the fused path: scores kept on chip, per-chunk candidates into
    `workspace`; with k_new / slot_mapping also this step's new K rows."""
    _score_candidates("idx_score_candidates", q_fp8, w, cache, batch, k, workspace, k_new,
                      slot_mapping, stream)


def idx_select_candidates(q_fp8, w, cache, batch, k, workspace, topk=None, stream=None):
    """Second launch of the fused path: each row's top k from the candidates."""
    return _select_candidates("idx_select_candidates", q_fp8, w, cache, batch, k, workspace, topk,
                              stream)


def idx_score_candidates_fp4(q_fp8, w, cache, batch, k, workspace, k_new=None, slot_mapping=None,
                             stream=None):
    """idx_score_candidates over an FP4 cache (a KCacheFP4)."""
    _score_candidates("idx_score_candidates_fp4", q_fp8, w, cache, batch, k, workspace, k_new,
                      slot_mapping, stream)


def idx_select_candidates_fp4(q_fp8, w, cache, batch, k, workspace, topk=None, stream=None):
    return _select_candidates("idx_select_candidates_fp4", q_fp8, w, cache, batch, k, workspace,
                              topk, stream)


NOALLOC_SCRATCH_BYTES = 32 << 20


def idx_score_topk_noalloc(q_fp8, w, cache, batch, k, topk, stream=None):
    """idx_score_topk with the library's own per-device scratch (no workspace argument)."""
    _check("idx_score_topk_noalloc",
           _lib.idx_score_topk_noalloc(_ptr(q_fp8), _ptr(w), N_HEADS, HEAD_DIM, cache.c(), batch.c(),
                                       k, _ptr(topk), int(topk.stride(0)), _stream(stream)))
    return topk


def idx_layer_schedule(use_index_cache, pattern, freq, offset, num_layers):
    """List of bools, True for F layers (host only)."""
    out = (ctypes.c_uint8 * max(num_layers, 1))()
    pat = None if pattern is None else pattern.encode()
    _check("idx_layer_schedule",
           _lib.idx_layer_schedule(int(use_index_cache), pat, int(freq), int(offset),
                                   int(num_layers), ctypes.cast(out, ctypes.c_void_p)))
    return [bool(out[i]) for i in range(num_layers)]


def _layer_io(k_new, cache, q_fp8, w):
    k_new = as_bf16_bits(k_new)
    return LayerIOC(k_new.data_ptr(), int(k_new.stride(0)), cache.c(),
                    0 if q_fp8 is None else q_fp8.data_ptr(), 0 if w is None else w.data_ptr())


def idx_indexcache_layer(k_new, cache, q_fp8, w, is_full, write_k, slot_mapping, batch, k, topk,
                         workspace=None, stream=None):
    io = _layer_io(k_new, cache, q_fp8, w)
    ws = _workspace(idx_score_topk_workspace_size(batch, k), topk.device, workspace)
    _check("idx_indexcache_layer",
           _lib.idx_indexcache_layer(ctypes.byref(io), int(is_full), int(write_k), _ptr(slot_mapping),
                                     batch.c(), k, _ptr(topk), int(topk.stride(0)), _ptr(ws),
                                     ws.numel(), _stream(stream)))


def idx_indexcache_layer_fp4(k_new, cache, q_fp8, w, is_full, write_k, slot_mapping, batch, k,
                             topk, workspace=None, stream=None):
    """idx_indexcache_layer over an FP4 cache (a KCacheFP4)."""
    io = _layer_io(k_new, cache, q_fp8, w)
    ws = _workspace(idx_score_topk_fp4_workspace_size(batch, k), topk.device, workspace)
    _check("idx_indexcache_layer_fp4",
           _lib.idx_indexcache_layer_fp4(ctypes.byref(io), int(is_full), int(write_k),
                                         _ptr(slot_mapping), batch.c(), k, _ptr(topk),
                                         int(topk.stride(0)), _ptr(ws), ws.numel(), _stream(stream)))


def idx_indexcache_stack(layers, is_full, write_k_on_s, slot_mapping, batch, k, topk,
                         workspace=None, stream=None):
    """layers: list of (k_new, cache, q_fp8, w); is_full: list of bools."""
    n = len(layers)
    arr = (LayerIOC * n)(*[_layer_io(*lay) for lay in layers])
    full = (ctypes.c_uint8 * n)(*[1 if f else 0 for f in is_full])
    ws = _workspace(idx_score_topk_workspace_size(batch, k), topk.device, workspace)
    _check("idx_indexcache_stack",
           _lib.idx_indexcache_stack(arr, n, ctypes.cast(full, ctypes.c_void_p), int(write_k_on_s),
                                     _ptr(slot_mapping), batch.c(), k, _ptr(topk),
                                     int(topk.stride(0)), _ptr(ws), ws.numel(), _stream(stream)))


class Physical:
    """The consumer's physical top-k rows and valid counts of an index group:
    [num_tokens, k] int32 rows over a pool of num_blocks blocks of block_size
    positions (physical slot = block * block_stride_rows + offset)."""

    def __init__(self, num_tokens, k, num_blocks, block_size=BLOCK_SIZE, block_stride_rows=0,
                 device="cuda", fill=None):
        self.physical = torch.empty((num_tokens, k), dtype=torch.int32, device=device)
        self.valid_counts = torch.empty((num_tokens,), dtype=torch.int32, device=device)
        if fill is not None:
            self.physical.fill_(fill)
            self.valid_counts.fill_(fill)
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.block_stride_rows = int(block_stride_rows)

    def c(self):
        return PhysicalC(_ptr(self.physical), int(self.physical.stride(0)), _ptr(self.valid_counts),
                         self.block_size, self.num_blocks, self.block_stride_rows)


def idx_indexcache_layer_physical(k_new, cache, q_fp8, w, is_full, write_k, slot_mapping, batch, k,
                                  topk, physical, workspace=None, stream=None):
    """idx_indexcache_layer that also converts an F layer's rows into `physical`
    (a Physical); S layers leave it alone."""
    io = _layer_io(k_new, cache, q_fp8, w)
    ph = physical.c()
    ws = _workspace(idx_score_topk_workspace_size(batch, k), topk.device, workspace)
    _check("idx_indexcache_layer_physical",
           _lib.idx_indexcache_layer_physical(ctypes.byref(io), int(is_full), int(write_k),
                                              _ptr(slot_mapping), batch.c(), k, _ptr(topk),
                                              int(topk.stride(0)), ctypes.byref(ph), _ptr(ws),
                                              ws.numel(), _stream(stream)))


def idx_indexcache_stack_physical(layers, is_full, write_k_on_s, slot_mapping, batch, k, topk,
                                  physical, workspace=None, stream=None):
    n = len(layers)
    arr = (LayerIOC * n)(*[_layer_io(*lay) for lay in layers])
    full = (ctypes.c_uint8 * n)(*[1 if f else 0 for f in is_full])
    ph = physical.c()
    ws = _workspace(idx_score_topk_workspace_size(batch, k), topk.device, workspace)
    _check("idx_indexcache_stack_physical",
           _lib.idx_indexcache_stack_physical(arr, n, ctypes.cast(full, ctypes.c_void_p),
                                              int(write_k_on_s), _ptr(slot_mapping), batch.c(), k,
                                              _ptr(topk), int(topk.stride(0)), ctypes.byref(ph),
                                              _ptr(ws), ws.numel(), _stream(stream)))


def idx_topk_to_physical(logical, batch, num_blocks, block_size=BLOCK_SIZE, block_stride_rows=0,
                         physical=None, valid_counts=None, stream=None):
    T, k = int(logical.shape[0]), int(logical.shape[1])
    if physical is None:
        physical = torch.empty((T, k), dtype=torch.int32, device=logical.device)
    if valid_counts is None:
        valid_counts = torch.empty((T,), dtype=torch.int32, device=logical.device)
    _check("idx_topk_to_physical",
           _lib.idx_topk_to_physical(_ptr(logical), int(logical.stride(0)), batch.c(), block_size,
                                     int(num_blocks), k, int(block_stride_rows), _ptr(physical),
                                     int(physical.stride(0)), _ptr(valid_counts), _stream(stream)))
    return physical, valid_counts


def _hip_runtime():
    """The HIP runtime this process already uses (torch's; libidx binds to it too)."""
    for line in open("/proc/self/maps"):
        path = line.split()[-1]
        if os.path.basename(path).startswith("libamdhip64.so"):
            lib = ctypes.CDLL(path)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            return lib
    raise RuntimeError("the HIP runtime is not loaded in this process")


_hip = None
# hipEventReleaseToDevice (a device-scope release when recorded), else
# hipEventDisableSystemFence; the two together are refused when recorded
_EVENT_FLAGS = (0x40000000, 0x20000000)


class HipEvent:
    """A HIP event for timing only, recorded with a device-scope release instead
    of the system-scope fence of a default event (a cache write-back and
    invalidate, which would add itself to every bracketed kernel)."""

    def __init__(self):
        global _hip
        if _hip is None:
            _hip = _hip_runtime()
        self.handle = ctypes.c_void_p()
        for flags in _EVENT_FLAGS:
            if _hip.hipEventCreateWithFlags(ctypes.byref(self.handle), flags) == 0:
                return
        raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        if _hip.hipEventRecord(self.handle, ctypes.c_void_p(s.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end):
        ms = ctypes.c_float()
        if _hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)


class KernelTrace:
    """Per-kernel times of the library calls made inside a ``with`` block on this
    thread (idx_trace_begin / idx_trace_end): ``kernels`` lists (name, ms) in
    launch order after the block, once the work has finished.  ``capacity`` is
    the number of kernels that can be timed."""

    def __init__(self, capacity=256, stream=None):
        self.capacity = int(capacity)
        self.stream = torch.cuda.current_stream() if stream is None else stream
        self.kernels = []

    def __enter__(self):
        self._events = [HipEvent() for _ in range(2 * self.capacity)]
        self._arr = (ctypes.c_void_p * len(self._events))(*[e.handle.value for e in self._events])
        _check("idx_trace_begin", _lib.idx_trace_begin(ctypes.cast(self._arr, ctypes.c_void_p),
                                                      len(self._events)))
        return self

    def __exit__(self, *exc):
        names = (ctypes.c_char_p * self.capacity)()
        n = _lib.idx_trace_end(ctypes.cast(names, ctypes.c_void_p), self.capacity)
        self.stream.synchronize()
        self.kernels = [(names[i].decode(), self._events[2 * i].elapsed_ms(self._events[2 * i + 1]))
                        for i in range(n)]
        return False

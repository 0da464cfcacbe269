"""MI355X (gfx950) DSA lightning indexer with IndexCache layer reuse.

The compute lives in libidx.so (hand-written HIP kernels behind a C ABI,
declared in include/idx.h); ``binding`` marshals torch tensors into it.
"""

from .binding import (  # noqa: F401
    Batch, HipEvent, IdxError, KCache, KCacheFP4, KernelTrace, Physical, idx_indexcache_layer,
    idx_indexcache_layer_fp4, idx_indexcache_layer_physical, idx_indexcache_stack,
    idx_indexcache_stack_physical,
    idx_layer_schedule, idx_logits, idx_logits_fp4, idx_quant_q_fold_w, idx_quant_write_k,
    idx_quant_write_k_fp4, idx_score_candidates, idx_score_candidates_fp4, idx_score_topk,
    idx_score_topk_fp4,
    idx_score_topk_fp4_workspace_size, idx_score_topk_noalloc, idx_score_topk_workspace_size,
    idx_select_candidates, idx_select_candidates_fp4,
    idx_topk, idx_topk_to_physical, idx_topk_workspace_size, idx_version, lib)

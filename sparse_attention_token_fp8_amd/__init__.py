"""MI355X (gfx950) DSA lightning indexer with IndexCache layer reuse.

The compute lives in libidx.so (hand-written HIP kernels behind a C ABI,
declared in include/idx.h); ``binding`` marshals torch tensors into it.
"""

from .binding import (Batch, HipEvent, IdxError, KCache, KernelTrace, idx_indexcache_layer,  # noqa: F401
                      idx_indexcache_stack, idx_layer_schedule, idx_logits, idx_quant_q_fold_w,
                      idx_quant_write_k, idx_score_candidates, idx_score_topk, idx_score_topk_noalloc,
                      idx_select_candidates,
                      idx_score_topk_workspace_size, idx_topk,
                      idx_topk_to_physical, idx_topk_workspace_size, idx_version, lib)

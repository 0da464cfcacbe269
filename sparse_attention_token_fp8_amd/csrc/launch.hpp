// Kernel launchers (internal).  Each enqueues on `stream` and returns the
// launch status; argument checking happens in api.cpp before any of these.
#pragma once

#include "common.hpp"

namespace idx {

// Tracing (idx_trace_begin): records the next caller event on `stream`
// before (after = false) or after (after = true) the kernel `name`; a no-op
// unless the calling thread is tracing.
void trace_mark(hipStream_t stream, const char* name, bool after);

// Every kernel launch of the library goes through this, so a trace sees it.
#define IDX_LAUNCH(NAME, KERNEL, GRID, BLOCK, STREAM, ...)                  \
  do {                                                                      \
    ::idx::trace_mark(STREAM, NAME, false);                                 \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);        \
    ::idx::trace_mark(STREAM, NAME, true);                                  \
  } while (0)

hipError_t launch_quant_write_k(const uint16_t* k, int64_t num_rows, int64_t stride,
                                const int64_t* slots, uint8_t* cache, int64_t num_slots,
                                hipStream_t stream);

hipError_t launch_quant_q_fold(const uint16_t* q, const float* w_raw, int64_t num_rows,
                               float softmax_scale, float head_norm, uint8_t* q8, float* w_out,
                               float* qs_out, hipStream_t stream);

// Scores into `logits` (row stride ld), and each row's sampled scores into
// samp[t][...] when samp is not null.  Tokens below dec_tokens use the
// decode work split (one token per work-group), the rest the prefill split; a
// batch whose requests have at most one new token each is all decode.
hipError_t launch_score(const uint8_t* q8, const float* w, const CacheArgs& cache,
                        const BatchArgs& b, int64_t dec_tokens, float* logits, int64_t ld,
                        float* samp, hipStream_t stream);

// The FP4 cache (4352-byte blocks): quantise-and-scatter, and scores (decode
// batches with the decode split, every other batch with the prefill split).
hipError_t launch_quant_write_k_fp4(const uint16_t* k, int64_t num_rows, int64_t stride,
                                    const int64_t* slots, uint8_t* cache, int64_t num_slots,
                                    hipStream_t stream);
hipError_t launch_score_fp4(const uint8_t* q8, const float* w, const CacheArgs& cache,
                            const BatchArgs& b, int64_t dec_tokens, float* logits, int64_t ld,
                            float* samp, hipStream_t stream);

// Blocks per decode work-group for `tokens` rows of up to max_seq_len
// positions (a multiple of 4, 8..64).
int decode_chunk_blocks(int max_seq_len, int64_t tokens);

// Whether launch_score_write_k can score this batch: every token scored with
// the decode split and at most a few new tokens per request.
bool score_writes_k(const BatchArgs& b, int64_t dec_tokens);

// Decode scoring that also quantises this step's new K rows (row t of k to
// slots[t]) into the cache, as launch_quant_write_k would before scoring.
// Rows whose slot is not the block-table slot of their position are written
// but not patched into the scores.
hipError_t launch_score_write_k(const uint8_t* q8, const float* w, const CacheArgs& cache,
                                const BatchArgs& b, const uint16_t* k, int64_t k_stride,
                                const int64_t* slots, uint8_t* cache_w, float* logits, int64_t ld,
                                float* samp, hipStream_t stream);

// Whether idx_score_topk takes the fused path for this batch: every token
// scored with the decode split, rows long enough for the long-row top-k.
bool keep_path(const BatchArgs& b, int64_t dec_tokens);

// Workspace of the fused path; returns its bytes and, with a base, fills `ks`.
size_t keep_workspace_layout(const BatchArgs& b, void* base, KeepSlots* ks);

// The fused path's two launches.  launch_keep_candidates scores the batch
// with the scores kept on chip and leaves each chunk's candidates in `ks`; with
// kq, this step's new K rows are written first (by the scoring kernel itself,
// so score_writes_k must hold).  launch_keep_select takes each row's top k
// from the candidates (rescoring a row whose chunks held more than their
// share).  fp4: the cache is the FP4 one (the same method and kernels, FP4
// block loads).
hipError_t launch_keep_candidates(const uint8_t* q8, const float* w, const CacheArgs& cache,
                                  const BatchArgs& b, const uint16_t* kq, int64_t kq_stride,
                                  const int64_t* slots, uint8_t* cache_w, int k,
                                  const KeepSlots& ks, hipStream_t stream, bool fp4 = false);
hipError_t launch_keep_select(const uint8_t* q8, const float* w, const CacheArgs& cache,
                              const BatchArgs& b, int k, const KeepSlots& ks, int32_t* out,
                              int64_t ldo, hipStream_t stream, bool fp4 = false);

// Finish long rows from the candidate slots of `ws`.
hipError_t launch_topk_resolve(const float* logits, int64_t ld, const BatchArgs& b,
                               const TopkWorkspace& ws, int k, int32_t* out, int64_t ldo,
                               hipStream_t stream);

// Top-k rows from scores (row stride ld) into out (row stride ldo).
hipError_t launch_topk(const float* logits, int64_t ld, const BatchArgs& b, const TopkWorkspace& ws,
                       int k, int32_t* out, int64_t ldo, hipStream_t stream);

hipError_t launch_topk_to_physical(const int32_t* logical, int64_t ldl, const BatchArgs& b,
                                   int block_size, int64_t num_blocks, int k, int64_t stride_rows,
                                   int32_t* physical, int64_t ldp, int32_t* valid,
                                   hipStream_t stream);

}  // namespace idx

// The C ABI of libidx: host-side argument checks, workspace carving and
// kernel dispatch.  Nothing here allocates, frees or synchronises.

#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

using namespace idx;

namespace {

constexpr int kMaxTokens = 65535;  // grid y-extent used for per-token launches

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

idx_status_t check_cache(const idx_kcache_t& c) {
  if (c.block_size != kBlock) return IDX_ERR_UNSUPPORTED;
  if (c.num_blocks < 0) return IDX_ERR_INVALID_ARG;
  if (c.num_blocks > 0 && (c.data == nullptr || !aligned(c.data, 16))) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

// block_size: positions per block-table entry (the cache's 64 for every
// scoring call; the caller's for the physical conversion).
idx_status_t check_batch(const idx_batch_t* b, int64_t block_size = kBlock) {
  if (b == nullptr) return IDX_ERR_INVALID_ARG;
  if (b->num_reqs < 1 || b->num_tokens < 0 || b->max_seq_len < 0 || b->max_query_len < 0)
    return IDX_ERR_INVALID_ARG;
  if (b->num_tokens > kMaxTokens || b->max_seq_len > topk_max_seq_len()) return IDX_ERR_UNSUPPORTED;
  if (b->seq_lens == nullptr || b->query_start_loc == nullptr || b->block_table == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (!aligned(b->seq_lens, 4) || !aligned(b->query_start_loc, 4) || !aligned(b->block_table, 4))
    return IDX_ERR_INVALID_ARG;
  if (block_size < 1 ||
      b->block_table_stride < ((int64_t)b->max_seq_len + block_size - 1) / block_size ||
      b->block_table_stride < 1)
    return IDX_ERR_INVALID_ARG;
  if (b->max_query_len > b->num_tokens) return IDX_ERR_INVALID_ARG;
  if (b->num_decode_tokens < 0 || b->num_decode_tokens > b->num_tokens) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

BatchArgs to_args(const idx_batch_t* b) {
  BatchArgs a;
  a.seq_lens = b->seq_lens;
  a.qsl = b->query_start_loc;
  a.bt = b->block_table;
  a.bt_stride = b->block_table_stride;
  a.num_reqs = b->num_reqs;
  a.num_tokens = b->num_tokens;
  a.max_seq_len = b->max_seq_len;
  a.max_query_len = b->max_query_len;
  return a;
}

idx_status_t check_scoring(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                           int32_t head_dim, const idx_kcache_t& cache, const idx_batch_t* b) {
  if (n_heads != kHeads || head_dim != kHeadDim) return IDX_ERR_UNSUPPORTED;
  idx_status_t s = check_cache(cache);
  if (s != IDX_OK) return s;
  s = check_batch(b);
  if (s != IDX_OK) return s;
  if (b->num_tokens > 0 && (q_fp8 == nullptr || w == nullptr)) return IDX_ERR_INVALID_ARG;
  if (!aligned(q_fp8, 16) || !aligned(w, 16)) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

idx_status_t check_k(int32_t k, int64_t topk_stride, const int32_t* topk, int32_t num_tokens) {
  if (k < 1 || k > kMaxK) return IDX_ERR_UNSUPPORTED;
  if (topk_stride < k) return IDX_ERR_INVALID_ARG;
  if (num_tokens > 0 && topk == nullptr) return IDX_ERR_INVALID_ARG;
  if (!aligned(topk, 4)) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

int64_t fused_ld(const idx_batch_t* b) {
  return (int64_t)align_up((size_t)std::max(b->max_seq_len, 1), (size_t)kBlock);
}

idx_status_t launched(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH; }

size_t fused_workspace(const idx_batch_t* b, void* base, TopkWorkspace* ws) {
  return topk_workspace_layout(b->num_tokens, b->max_seq_len, fused_ld(b), base, ws);
}

idx_status_t check_k_rows(const uint16_t* k_bf16, int64_t k_row_stride, const int64_t* slot_mapping,
                          const idx_kcache_t& cache, int64_t num_tokens) {
  if (num_tokens == 0) return IDX_OK;
  if (k_bf16 == nullptr || slot_mapping == nullptr || cache.data == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (k_row_stride < kHeadDim || (k_row_stride % 4) != 0 || !aligned(k_bf16, 8) ||
      !aligned(slot_mapping, 8))
    return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

// The fused path's first launch (scores kept on chip, each chunk's candidates
// into the workspace); with kq set, this step's new K rows are quantised into
// the cache first (by the scoring kernel itself when the batch allows it).
hipError_t keep_candidates(const uint8_t* q_fp8, const float* w, const idx_kcache_t& cache,
                           const idx_batch_t* batch, int32_t k, void* workspace,
                           const uint16_t* kq, int64_t kq_stride, const int64_t* slots,
                           hipStream_t stream, bool fp4 = false) {
  const BatchArgs b = to_args(batch);
  KeepSlots ks;
  keep_workspace_layout(b, workspace, &ks);
  const bool fk = kq != nullptr && score_writes_k(b, batch->num_decode_tokens);
  if (kq != nullptr && !fk) {
    const int64_t ns = cache.num_blocks * kBlock;
    const hipError_t e =
        fp4 ? launch_quant_write_k_fp4(kq, batch->num_tokens, kq_stride, slots, cache.data, ns, stream)
            : launch_quant_write_k(kq, batch->num_tokens, kq_stride, slots, cache.data, ns, stream);
    if (e != hipSuccess) return e;
  }
  return launch_keep_candidates(q_fp8, w, CacheArgs{cache.data, cache.num_blocks}, b,
                                fk ? kq : nullptr, kq_stride, slots, cache.data, k, ks, stream,
                                fp4);
}

// Scores + top-k of one batch into `topk`; with kq set, this step's new K rows
// are quantised into the cache first (by the decode scoring kernel itself
// when it scores the whole batch).  Arguments are already checked.
hipError_t score_topk(const uint8_t* q_fp8, const float* w, const idx_kcache_t& cache,
                      const idx_batch_t* batch, int32_t k, int32_t* topk, int64_t topk_stride,
                      void* workspace, const uint16_t* kq, int64_t kq_stride,
                      const int64_t* slots, hipStream_t stream) {
  if (keep_path(to_args(batch), batch->num_decode_tokens)) {
    hipError_t e = keep_candidates(q_fp8, w, cache, batch, k, workspace, kq, kq_stride, slots,
                                   stream);
    if (e != hipSuccess) return e;
    KeepSlots ks;
    keep_workspace_layout(to_args(batch), workspace, &ks);
    return launch_keep_select(q_fp8, w, CacheArgs{cache.data, cache.num_blocks}, to_args(batch), k,
                              ks, topk, topk_stride, stream);
  }
  TopkWorkspace ws;
  fused_workspace(batch, workspace, &ws);
  const BatchArgs b = to_args(batch);
  const CacheArgs c{cache.data, cache.num_blocks};
  hipError_t e = hipSuccess;
  if (kq != nullptr && score_writes_k(b, batch->num_decode_tokens)) {
    e = launch_score_write_k(q_fp8, w, c, b, kq, kq_stride, slots, cache.data, ws.logits, ws.ld,
                             ws.samp, stream);
  } else {
    if (kq != nullptr)
      e = launch_quant_write_k(kq, batch->num_tokens, kq_stride, slots, cache.data,
                               cache.num_blocks * kBlock, stream);
    if (e == hipSuccess)
      e = launch_score(q_fp8, w, c, b, batch->num_decode_tokens, ws.logits, ws.ld, ws.samp, stream);
  }
  if (e == hipSuccess) e = launch_topk(ws.logits, ws.ld, b, ws, k, topk, topk_stride, stream);
  return e;
}

// Every layer of a stack, checked before anything is enqueued.
idx_status_t check_stack(const idx_layer_io_t* layers, int32_t num_layers, const uint8_t* is_full,
                         int32_t write_k_on_s, const int64_t* slot_mapping,
                         const idx_batch_t* batch, int32_t k, const int32_t* topk,
                         int64_t topk_stride, const void* workspace, size_t workspace_bytes) {
  if (layers == nullptr || is_full == nullptr || num_layers < 1) return IDX_ERR_INVALID_ARG;
  if (!is_full[0]) return IDX_ERR_INVALID_ARG;
  idx_status_t s = check_batch(batch);
  if (s != IDX_OK) return s;
  for (int l = 0; l < num_layers; ++l) {
    const idx_layer_io_t& L = layers[l];
    s = check_cache(L.cache);
    if (s != IDX_OK) return s;
    if (is_full[l]) {
      s = check_scoring(L.q_fp8, L.w, kHeads, kHeadDim, L.cache, batch);
      if (s != IDX_OK) return s;
    }
    if ((is_full[l] || write_k_on_s) && batch->num_tokens > 0 &&
        (L.k_bf16 == nullptr || L.k_row_stride < kHeadDim || (L.k_row_stride % 4) != 0 ||
         !aligned(L.k_bf16, 8) || slot_mapping == nullptr || !aligned(slot_mapping, 8) ||
         L.cache.data == nullptr))
      return IDX_ERR_INVALID_ARG;
  }
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens > 0 &&
      (workspace == nullptr || workspace_bytes < idx_score_topk_workspace_size(batch, k) ||
       !aligned(workspace, 256)))
    return IDX_ERR_WORKSPACE;
  return IDX_OK;
}

// The physical conversion's arguments (the consumer's block size, pool and
// output rows) for rows of k entries.
idx_status_t check_physical(const idx_batch_t* batch, int32_t k, const idx_physical_t* p) {
  if (p->block_size < 1) return IDX_ERR_INVALID_ARG;
  idx_status_t s = check_batch(batch, p->block_size);
  if (s != IDX_OK) return s;
  if (k < 1 || k > kMaxK) return IDX_ERR_UNSUPPORTED;
  if (p->num_blocks < 0 || p->block_stride_rows < 0) return IDX_ERR_INVALID_ARG;
  const int64_t stride_rows = p->block_stride_rows ? p->block_stride_rows : p->block_size;
  if (stride_rows < p->block_size) return IDX_ERR_INVALID_ARG;
  if (p->num_blocks * stride_rows > (int64_t)INT32_MAX) return IDX_ERR_UNSUPPORTED;
  if (p->physical_stride < k) return IDX_ERR_INVALID_ARG;
  if (batch->num_tokens > 0 && p->physical == nullptr) return IDX_ERR_INVALID_ARG;
  if (!aligned(p->physical, 4) || !aligned(p->valid_counts, 4)) return IDX_ERR_INVALID_ARG;
  return IDX_OK;
}

hipError_t to_physical(const int32_t* logical, int64_t logical_stride, const idx_batch_t* batch,
                       int32_t k, const idx_physical_t& p, hipStream_t stream) {
  const int64_t stride_rows = p.block_stride_rows ? p.block_stride_rows : p.block_size;
  return launch_topk_to_physical(logical, logical_stride, to_args(batch), p.block_size,
                                 p.num_blocks, k, stride_rows, p.physical, p.physical_stride,
                                 p.valid_counts, stream);
}

}  // namespace

// Workspace of idx_score_topk_noalloc, for callers that cannot allocate: one
// copy of this array per device, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it passes the device address looked up once per
// device by noalloc_scratch().
static __device__ __align__(256) uint8_t scratch[IDX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch`, looked up on the first call per device
// (with that device current); nullptr if the lookup fails.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

const char* idx_status_str(idx_status_t s) {
  switch (s) {
    case IDX_OK: return "ok";
    case IDX_ERR_INVALID_ARG: return "invalid argument";
    case IDX_ERR_UNSUPPORTED: return "unsupported shape";
    case IDX_ERR_WORKSPACE: return "workspace missing or too small";
    case IDX_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* idx_version(void) { return "idx 0.1 gfx950"; }

idx_status_t idx_quant_write_k(const uint16_t* k_bf16, int64_t num_tokens, int32_t head_dim,
                               int64_t k_row_stride, const int64_t* slot_mapping,
                               idx_kcache_t cache, hipStream_t stream) {
  if (head_dim != kHeadDim) return IDX_ERR_UNSUPPORTED;
  idx_status_t s = check_cache(cache);
  if (s != IDX_OK) return s;
  if (num_tokens < 0) return IDX_ERR_INVALID_ARG;
  if (num_tokens == 0) return IDX_OK;
  if (k_bf16 == nullptr || slot_mapping == nullptr || cache.data == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (k_row_stride < head_dim || (k_row_stride % 4) != 0 || !aligned(k_bf16, 8) ||
      !aligned(slot_mapping, 8))
    return IDX_ERR_INVALID_ARG;
  return launched(launch_quant_write_k(k_bf16, num_tokens, k_row_stride, slot_mapping, cache.data,
                                       cache.num_blocks * kBlock, stream));
}

idx_status_t idx_quant_q_fold_w(const uint16_t* q_bf16, const float* w_raw, int64_t num_tokens,
                                int32_t n_heads, int32_t head_dim, float softmax_scale,
                                uint8_t* q_fp8, float* w_folded, float* q_scale_out,
                                hipStream_t stream) {
  if (n_heads != kHeads || head_dim != kHeadDim) return IDX_ERR_UNSUPPORTED;
  if (num_tokens < 0) return IDX_ERR_INVALID_ARG;
  if (num_tokens == 0) return IDX_OK;
  if (q_bf16 == nullptr || w_raw == nullptr || q_fp8 == nullptr || w_folded == nullptr)
    return IDX_ERR_INVALID_ARG;
  if (!aligned(q_bf16, 8) || !aligned(q_fp8, 16) || !aligned(w_raw, 4) || !aligned(w_folded, 4) ||
      !aligned(q_scale_out, 4))
    return IDX_ERR_INVALID_ARG;
  const float head_norm = (float)(1.0 / __builtin_sqrt((double)n_heads));
  return launched(launch_quant_q_fold(q_bf16, w_raw, num_tokens * n_heads, softmax_scale,
                                      head_norm, q_fp8, w_folded, q_scale_out, stream));
}

idx_status_t idx_logits(const uint8_t* q_fp8, const float* w, int32_t n_heads, int32_t head_dim,
                        idx_kcache_t cache, const idx_batch_t* batch, float* logits,
                        int64_t logits_stride, hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (logits == nullptr || logits_stride < batch->max_seq_len || !aligned(logits, 4))
    return IDX_ERR_INVALID_ARG;
  CacheArgs c{cache.data, cache.num_blocks};
  return launched(launch_score(q_fp8, w, c, to_args(batch), batch->num_decode_tokens, logits,
                               logits_stride, nullptr, stream));
}

size_t idx_topk_workspace_size(const idx_batch_t* batch, int32_t k) {
  if (batch == nullptr || batch->num_tokens <= 0 || k < 1) return 0;
  return topk_workspace_layout(batch->num_tokens, batch->max_seq_len, 0, nullptr, nullptr);
}

idx_status_t idx_topk(const float* logits, int64_t logits_stride, const idx_batch_t* batch,
                      int32_t k, int32_t* topk, int64_t topk_stride, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  idx_status_t s = check_batch(batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (logits == nullptr || logits_stride < batch->max_seq_len || !aligned(logits, 4))
    return IDX_ERR_INVALID_ARG;
  const size_t need = idx_topk_workspace_size(batch, k);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  TopkWorkspace ws;
  topk_workspace_layout(batch->num_tokens, batch->max_seq_len, 0, workspace, &ws);
  return launched(launch_topk(logits, logits_stride, to_args(batch), ws, k, topk, topk_stride,
                              stream));
}

size_t idx_score_topk_workspace_size(const idx_batch_t* batch, int32_t k) {
  if (batch == nullptr || batch->num_tokens <= 0 || k < 1) return 0;
  if (check_batch(batch) != IDX_OK) return 0;
  if (keep_path(to_args(batch), batch->num_decode_tokens))
    return keep_workspace_layout(to_args(batch), nullptr, nullptr);
  return fused_workspace(batch, nullptr, nullptr);
}

idx_status_t idx_quant_write_k_fp4(const uint16_t* k_bf16, int64_t num_tokens, int32_t head_dim,
                                   int64_t k_row_stride, const int64_t* slot_mapping,
                                   idx_kcache_t cache, hipStream_t stream) {
  if (head_dim != kHeadDim) return IDX_ERR_UNSUPPORTED;
  idx_status_t s = check_cache(cache);
  if (s != IDX_OK) return s;
  if (num_tokens < 0) return IDX_ERR_INVALID_ARG;
  if (num_tokens == 0) return IDX_OK;
  s = check_k_rows(k_bf16, k_row_stride, slot_mapping, cache, num_tokens);
  if (s != IDX_OK) return s;
  return launched(launch_quant_write_k_fp4(k_bf16, num_tokens, k_row_stride, slot_mapping,
                                           cache.data, cache.num_blocks * kBlock, stream));
}

idx_status_t idx_logits_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads, int32_t head_dim,
                            idx_kcache_t cache, const idx_batch_t* batch, float* logits,
                            int64_t logits_stride, hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (logits == nullptr || logits_stride < batch->max_seq_len || !aligned(logits, 4))
    return IDX_ERR_INVALID_ARG;
  return launched(launch_score_fp4(q_fp8, w, CacheArgs{cache.data, cache.num_blocks},
                                   to_args(batch), batch->num_decode_tokens, logits, logits_stride,
                                   nullptr, stream));
}

size_t idx_score_topk_fp4_workspace_size(const idx_batch_t* batch, int32_t k) {
  if (batch == nullptr || batch->num_tokens <= 0 || k < 1) return 0;
  if (check_batch(batch) != IDX_OK) return 0;
  if (keep_path(to_args(batch), batch->num_decode_tokens))
    return keep_workspace_layout(to_args(batch), nullptr, nullptr);
  return fused_workspace(batch, nullptr, nullptr);
}

}  // extern "C"

namespace {

// idx_score_topk_fp4's work (arguments already checked): decode batches over
// long rows take the fused path with the FP4 scoring kernel (the new K rows,
// with kq, written inside it when the batch allows), the others the FP4 scores
// into the workspace and the unfused top-k.
hipError_t score_topk_fp4(const uint8_t* q_fp8, const float* w, const idx_kcache_t& cache,
                          const idx_batch_t* batch, int32_t k, int32_t* topk, int64_t topk_stride,
                          void* workspace, const uint16_t* kq, int64_t kq_stride,
                          const int64_t* slots, hipStream_t stream) {
  const BatchArgs b = to_args(batch);
  const CacheArgs c{cache.data, cache.num_blocks};
  if (keep_path(b, batch->num_decode_tokens)) {
    hipError_t e = keep_candidates(q_fp8, w, cache, batch, k, workspace, kq, kq_stride, slots,
                                   stream, true);
    if (e != hipSuccess) return e;
    KeepSlots ks;
    keep_workspace_layout(b, workspace, &ks);
    return launch_keep_select(q_fp8, w, c, b, k, ks, topk, topk_stride, stream, true);
  }
  hipError_t e = hipSuccess;
  if (kq != nullptr)
    e = launch_quant_write_k_fp4(kq, batch->num_tokens, kq_stride, slots, cache.data,
                                 cache.num_blocks * kBlock, stream);
  if (e != hipSuccess) return e;
  TopkWorkspace ws;
  fused_workspace(batch, workspace, &ws);
  e = launch_score_fp4(q_fp8, w, c, b, batch->num_decode_tokens, ws.logits, ws.ld, ws.samp, stream);
  if (e == hipSuccess) e = launch_topk(ws.logits, ws.ld, b, ws, k, topk, topk_stride, stream);
  return e;
}

}  // namespace

extern "C" {

idx_status_t idx_score_topk_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                int32_t k, int32_t* topk, int64_t topk_stride, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (workspace == nullptr || workspace_bytes < idx_score_topk_fp4_workspace_size(batch, k) ||
      !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  return launched(score_topk_fp4(q_fp8, w, cache, batch, k, topk, topk_stride, workspace, nullptr,
                                 0, nullptr, stream));
}

idx_status_t idx_indexcache_layer_fp4(const idx_layer_io_t* layer, int32_t is_full,
                                      int32_t write_k, const int64_t* slot_mapping,
                                      const idx_batch_t* batch, int32_t k, int32_t* topk,
                                      int64_t topk_stride, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (layer == nullptr) return IDX_ERR_INVALID_ARG;
  idx_status_t s = check_batch(batch);
  if (s != IDX_OK) return s;
  if (!is_full) {
    if (!write_k) return IDX_OK;
    return idx_quant_write_k_fp4(layer->k_bf16, batch->num_tokens, kHeadDim, layer->k_row_stride,
                                 slot_mapping, layer->cache, stream);
  }
  s = check_scoring(layer->q_fp8, layer->w, kHeads, kHeadDim, layer->cache, batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  s = check_k_rows(layer->k_bf16, layer->k_row_stride, slot_mapping, layer->cache,
                   batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (workspace == nullptr || workspace_bytes < idx_score_topk_fp4_workspace_size(batch, k) ||
      !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  return launched(score_topk_fp4(layer->q_fp8, layer->w, layer->cache, batch, k, topk, topk_stride,
                                 workspace, layer->k_bf16, layer->k_row_stride, slot_mapping,
                                 stream));
}

idx_status_t idx_score_topk(const uint8_t* q_fp8, const float* w, int32_t n_heads, int32_t head_dim,
                            idx_kcache_t cache, const idx_batch_t* batch, int32_t k,
                            int32_t* topk, int64_t topk_stride, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  const size_t need = idx_score_topk_workspace_size(batch, k);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  return launched(score_topk(q_fp8, w, cache, batch, k, topk, topk_stride, workspace, nullptr, 0,
                             nullptr, stream));
}

idx_status_t idx_score_topk_noalloc(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                    int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                    int32_t k, int32_t* topk, int64_t topk_stride,
                                    hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (idx_score_topk_workspace_size(batch, k) > (size_t)IDX_NOALLOC_SCRATCH_BYTES)
    return IDX_ERR_WORKSPACE;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return IDX_ERR_LAUNCH;
  return launched(score_topk(q_fp8, w, cache, batch, k, topk, topk_stride, ws, nullptr, 0,
                             nullptr, stream));
}

}  // extern "C"

namespace {

idx_status_t score_candidates(bool fp4, const uint8_t* q_fp8, const float* w, int32_t n_heads,
                              int32_t head_dim, const idx_kcache_t& cache, const idx_batch_t* batch,
                              int32_t k, const uint16_t* k_bf16, int64_t k_row_stride,
                              const int64_t* slot_mapping, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  if (k < 1 || k > kMaxK) return IDX_ERR_UNSUPPORTED;
  if (batch->num_tokens == 0) return IDX_OK;
  if (!keep_path(to_args(batch), batch->num_decode_tokens)) return IDX_ERR_UNSUPPORTED;
  if (k_bf16 != nullptr) {
    s = check_k_rows(k_bf16, k_row_stride, slot_mapping, cache, batch->num_tokens);
    if (s != IDX_OK) return s;
  }
  if (workspace == nullptr ||
      workspace_bytes < keep_workspace_layout(to_args(batch), nullptr, nullptr) ||
      !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  return launched(keep_candidates(q_fp8, w, cache, batch, k, workspace, k_bf16, k_row_stride,
                                  slot_mapping, stream, fp4));
}

idx_status_t select_candidates(bool fp4, const uint8_t* q_fp8, const float* w, int32_t n_heads,
                               int32_t head_dim, const idx_kcache_t& cache,
                               const idx_batch_t* batch, int32_t k, int32_t* topk,
                               int64_t topk_stride, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  idx_status_t s = check_scoring(q_fp8, w, n_heads, head_dim, cache, batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (!keep_path(to_args(batch), batch->num_decode_tokens)) return IDX_ERR_UNSUPPORTED;
  if (workspace == nullptr ||
      workspace_bytes < keep_workspace_layout(to_args(batch), nullptr, nullptr) ||
      !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  KeepSlots ks;
  keep_workspace_layout(to_args(batch), workspace, &ks);
  return launched(launch_keep_select(q_fp8, w, CacheArgs{cache.data, cache.num_blocks},
                                     to_args(batch), k, ks, topk, topk_stride, stream, fp4));
}

}  // namespace

extern "C" {

idx_status_t idx_score_candidates(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                  int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                  int32_t k, const uint16_t* k_bf16, int64_t k_row_stride,
                                  const int64_t* slot_mapping, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return score_candidates(false, q_fp8, w, n_heads, head_dim, cache, batch, k, k_bf16,
                          k_row_stride, slot_mapping, workspace, workspace_bytes, stream);
}

idx_status_t idx_select_candidates(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                   int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                   int32_t k, int32_t* topk, int64_t topk_stride, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return select_candidates(false, q_fp8, w, n_heads, head_dim, cache, batch, k, topk, topk_stride,
                           workspace, workspace_bytes, stream);
}

idx_status_t idx_score_candidates_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                      int32_t head_dim, idx_kcache_t cache,
                                      const idx_batch_t* batch, int32_t k, const uint16_t* k_bf16,
                                      int64_t k_row_stride, const int64_t* slot_mapping,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return score_candidates(true, q_fp8, w, n_heads, head_dim, cache, batch, k, k_bf16,
                          k_row_stride, slot_mapping, workspace, workspace_bytes, stream);
}

idx_status_t idx_select_candidates_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                       int32_t head_dim, idx_kcache_t cache,
                                       const idx_batch_t* batch, int32_t k, int32_t* topk,
                                       int64_t topk_stride, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return select_candidates(true, q_fp8, w, n_heads, head_dim, cache, batch, k, topk, topk_stride,
                           workspace, workspace_bytes, stream);
}

idx_status_t idx_indexcache_layer(const idx_layer_io_t* layer, int32_t is_full, int32_t write_k,
                                  const int64_t* slot_mapping, const idx_batch_t* batch, int32_t k,
                                  int32_t* topk, int64_t topk_stride, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (layer == nullptr) return IDX_ERR_INVALID_ARG;
  idx_status_t s = check_batch(batch);
  if (s != IDX_OK) return s;
  if (!is_full) {
    if (!write_k) return IDX_OK;
    return idx_quant_write_k(layer->k_bf16, batch->num_tokens, kHeadDim, layer->k_row_stride,
                             slot_mapping, layer->cache, stream);
  }
  s = check_scoring(layer->q_fp8, layer->w, kHeads, kHeadDim, layer->cache, batch);
  if (s != IDX_OK) return s;
  s = check_k(k, topk_stride, topk, batch->num_tokens);
  if (s != IDX_OK) return s;
  s = check_k_rows(layer->k_bf16, layer->k_row_stride, slot_mapping, layer->cache,
                   batch->num_tokens);
  if (s != IDX_OK) return s;
  if (batch->num_tokens == 0) return IDX_OK;
  if (workspace == nullptr || workspace_bytes < idx_score_topk_workspace_size(batch, k) ||
      !aligned(workspace, 256))
    return IDX_ERR_WORKSPACE;
  return launched(score_topk(layer->q_fp8, layer->w, layer->cache, batch, k, topk, topk_stride,
                             workspace, layer->k_bf16, layer->k_row_stride, slot_mapping, stream));
}

idx_status_t idx_indexcache_stack(const idx_layer_io_t* layers, int32_t num_layers,
                                  const uint8_t* is_full, int32_t write_k_on_s,
                                  const int64_t* slot_mapping, const idx_batch_t* batch, int32_t k,
                                  int32_t* topk, int64_t topk_stride, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return idx_indexcache_stack_physical(layers, num_layers, is_full, write_k_on_s, slot_mapping,
                                       batch, k, topk, topk_stride, nullptr, workspace,
                                       workspace_bytes, stream);
}

idx_status_t idx_topk_to_physical(const int32_t* logical, int64_t logical_stride,
                                  const idx_batch_t* batch, int32_t block_size, int64_t num_blocks,
                                  int32_t k, int64_t block_stride_rows, int32_t* physical,
                                  int64_t physical_stride, int32_t* valid_counts,
                                  hipStream_t stream) {
  const idx_physical_t ph{physical, physical_stride, valid_counts, block_size, num_blocks,
                          block_stride_rows};
  idx_status_t s = check_physical(batch, k, &ph);
  if (s != IDX_OK) return s;
  if (logical_stride < k) return IDX_ERR_INVALID_ARG;
  if (batch->num_tokens == 0) return IDX_OK;
  if (logical == nullptr || !aligned(logical, 4)) return IDX_ERR_INVALID_ARG;
  return launched(to_physical(logical, logical_stride, batch, k, ph, stream));
}

idx_status_t idx_indexcache_layer_physical(const idx_layer_io_t* layer, int32_t is_full,
                                           int32_t write_k, const int64_t* slot_mapping,
                                           const idx_batch_t* batch, int32_t k, int32_t* topk,
                                           int64_t topk_stride, const idx_physical_t* phys,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  if (phys != nullptr && is_full) {
    const idx_status_t s = check_physical(batch, k, phys);
    if (s != IDX_OK) return s;
  }
  const idx_status_t s = idx_indexcache_layer(layer, is_full, write_k, slot_mapping, batch, k,
                                              topk, topk_stride, workspace, workspace_bytes,
                                              stream);
  if (s != IDX_OK || phys == nullptr || !is_full || batch->num_tokens == 0) return s;
  return launched(to_physical(topk, topk_stride, batch, k, *phys, stream));
}

idx_status_t idx_indexcache_stack_physical(const idx_layer_io_t* layers, int32_t num_layers,
                                           const uint8_t* is_full, int32_t write_k_on_s,
                                           const int64_t* slot_mapping, const idx_batch_t* batch,
                                           int32_t k, int32_t* topk, int64_t topk_stride,
                                           const idx_physical_t* phys, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (phys != nullptr) {
    const idx_status_t s = check_physical(batch, k, phys);
    if (s != IDX_OK) return s;
  }
  idx_status_t s = check_stack(layers, num_layers, is_full, write_k_on_s, slot_mapping, batch, k,
                               topk, topk_stride, workspace, workspace_bytes);
  if (s != IDX_OK) return s;
  for (int l = 0; l < num_layers; ++l) {
    s = idx_indexcache_layer_physical(&layers[l], is_full[l], write_k_on_s, slot_mapping, batch,
                                      k, topk, topk_stride, phys, workspace, workspace_bytes,
                                      stream);
    if (s != IDX_OK) return s;
  }
  return IDX_OK;
}

}  // extern "C"

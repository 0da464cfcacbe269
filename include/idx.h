/*
 * idx.h -- C ABI of libidx, an MI355X (gfx950) implementation of the
 * DeepSeek-V3.2 DSA lightning-indexer path with IndexCache layer reuse.
 *
 * Sources (web pages; cited by title and snippet / section):
 *   [blog]  "IndexCache: cross-layer index reuse in DeepSeek sparse attention"
 *           (atomage.cn) -- vLLM snippets DeepseekV32IndexerCache,
 *           DeepseekV32IndexerBackend, Indexer.forward, SparseAttnIndexer,
 *           the op body, DeepseekV32IndexerMetadata, the skip_topk schedule,
 *           the top-k buffer allocation, the MLA forward.
 *   [pr]    "PR #37735 report: [Feature]: IndexCache support for DSA models"
 *           (prhub.com.cn) -- Implementation, Key source snippets, Risks & impact.
 *   [group] vLLM API page "vllm.v1.attention.backends.mla.index_group" --
 *           SparseMLAIndexGroup, SparseMLAIndexGroupBuilder.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; scratch memory is passed in as
 *     a caller-owned workspace whose size the *_workspace_size calls report.
 *   - Every call validates its arguments on the host first.  A non-zero
 *     status means nothing was enqueued.  Device arrays must be aligned to
 *     their element size (int32 / fp32 to 4 bytes, int64 to 8, bf16 rows to
 *     8), q_fp8 and the cache to 16, workspaces to 256; a misaligned pointer
 *     is IDX_ERR_INVALID_ARG (IDX_ERR_WORKSPACE for a workspace).  Otherwise the kernels are enqueued
 *     on `stream` and the call returns at once; a failure inside a kernel
 *     surfaces at the caller's next synchronisation as a HIP error.
 *   - Kernels bound every memory access by the host-side sizes they are given
 *     (num_blocks, block_table_stride, max_seq_len, strides).  Device metadata
 *     that disagrees with them (a block id outside the pool, a sequence longer
 *     than max_seq_len) gives unspecified values for the affected positions
 *     but no out-of-bounds access.
 *   - Supported shapes: n_heads == 64, head_dim == 128, block_size == 64,
 *     1 <= k <= 2048.  Anything else returns IDX_ERR_UNSUPPORTED.
 *   - Calls are stream-ordered; calls on different streams that share a
 *     cache, buffer or workspace race.
 */
#ifndef IDX_H_
#define IDX_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum idx_status {
  IDX_OK = 0,
  IDX_ERR_INVALID_ARG = -1,  /* null pointer, negative size, stride too small, misaligned */
  IDX_ERR_UNSUPPORTED = -2,  /* a shape outside the supported set above */
  IDX_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  IDX_ERR_LAUNCH = -4        /* the HIP runtime refused a launch */
} idx_status_t;

/* Static, NUL-terminated description of a status code. */
const char* idx_status_str(idx_status_t s);

/* Library version string, e.g. "idx 0.1 gfx950". */
const char* idx_version(void);

/*
 * Paged indexer K cache ([blog] DeepseekV32IndexerCache,
 * DeepseekV32IndexerBackend.get_kv_cache_shape, "FP8 naive cache"):
 * uint8 [num_blocks, block_size, 132], one shared K per position (no V,
 * one KV head).  Byte order inside a block of B = block_size * 132 bytes:
 *   bytes [0, block_size*128)           128 E4M3 codes of offsets 0..block_size-1
 *   bytes [block_size*128, B)           one fp32 (little-endian) scale per offset
 * so the token at slot = block * block_size + off has its codes at
 * block*B + off*128 and its scale at block*B + block_size*128 + off*4.
 */
typedef struct idx_kcache {
  uint8_t* data;        /* device, num_blocks * block_size * 132 bytes, 16-byte aligned */
  int64_t num_blocks;
  int32_t block_size;   /* must be 64 */
} idx_kcache_t;

/*
 * One batch of query tokens ([blog] DeepseekV32IndexerMetadata: seq_lens,
 * max_seq_len, slot_mapping, decode/prefill counts; the paged backend's block
 * table).  Request r has seq_lens[r] positions in total, of which the last
 * n_r = query_start_loc[r+1] - query_start_loc[r] are this step's new
 * tokens; query token t = query_start_loc[r] + i sits at position
 * p_t = seq_lens[r] - n_r + i and is scored against positions 0..p_t.
 *
 * num_decode_tokens (the metadata's decode count, decodes listed first) only
 * chooses how scoring work is split, never the result: tokens
 * 0..num_decode_tokens-1 are scored one token per work-group (the split for
 * short queries over long contexts), the others in groups of consecutive
 * tokens of one request (the split for prefill chunks), both kinds in one
 * launch.  0 lets the library choose: the decode split when every request
 * has at most one new token, else the prefill split for all.
 */
typedef struct idx_batch {
  const int32_t* seq_lens;         /* device [num_reqs] */
  const int32_t* query_start_loc;  /* device [num_reqs + 1], query_start_loc[0] == 0 */
  const int32_t* block_table;      /* device [num_reqs, block_table_stride] physical block ids */
  int64_t block_table_stride;      /* >= ceil(max_seq_len / block_size) */
  int32_t num_reqs;                /* >= 1 */
  int32_t num_tokens;              /* host copy of query_start_loc[num_reqs] */
  int32_t max_seq_len;             /* host copy of max(seq_lens) */
  int32_t max_query_len;           /* host copy of max(n_r) */
  int32_t num_decode_tokens;       /* 0..num_tokens, see above */
} idx_batch_t;

/*
 * Quantise new K rows to E4M3 with one power-of-two fp32 scale per row and
 * scatter them into the paged cache ([blog] op body:
 * ops.indexer_k_quant_and_cache(k, kv_cache, slot_mapping, quant_block_size,
 * scale_fmt); "FP8 naive cache": 128 bytes + 4-byte fp32 scale).
 *   k_bf16        device bf16 bit patterns, row i at k_bf16 + i*k_row_stride,
 *                 head_dim values; 8-byte aligned, k_row_stride % 4 == 0
 *   slot_mapping  device int64 [num_tokens]; slot < 0 = padding, skipped;
 *                 slot >= num_blocks*block_size is skipped too
 * Per row: amax = max(max|x|, 1e-4); scale = smallest 2^e with
 * amax <= 448 * 2^e; code_i = E4M3(x_i / scale) rounded to nearest, ties to
 * even, sign of zero kept.  Only the bytes of the written slots change.
 * num_tokens == 0 is a no-op.
 */
idx_status_t idx_quant_write_k(const uint16_t* k_bf16, int64_t num_tokens, int32_t head_dim,
                               int64_t k_row_stride, const int64_t* slot_mapping,
                               idx_kcache_t cache, hipStream_t stream);

/*
 * Quantise q per (token, head) group of 128 with power-of-two scales and fold
 * the weights ([blog] Indexer.forward: per_token_group_quant_fp8(...,
 * use_ue8m0=True), then weights * q_scale * softmax_scale * n_head^-0.5).
 *   q_bf16        device bf16 bits [num_tokens, n_heads, head_dim], contiguous
 *   w_raw         device fp32 [num_tokens, n_heads]
 *   q_fp8         device out uint8 [num_tokens, n_heads, head_dim], 16-byte aligned
 *   w_folded      device out fp32 [num_tokens, n_heads]:
 *                 ((w_raw * q_scale) * softmax_scale) * n_heads^-0.5, fp32
 *   q_scale_out   device out fp32 [num_tokens, n_heads], or NULL
 * The quantiser is the one idx_quant_write_k uses.
 */
idx_status_t idx_quant_q_fold_w(const uint16_t* q_bf16, const float* w_raw, int64_t num_tokens,
                                int32_t n_heads, int32_t head_dim, float softmax_scale,
                                uint8_t* q_fp8, float* w_folded, float* q_scale_out,
                                hipStream_t stream);

/*
 * Lightning-indexer scores ([blog] SparseAttnIndexer / op body: fp8 q of 64
 * heads, one shared fp8 K per position, folded fp32 weights):
 *   logits[t*logits_stride + s] = ks[s] * sum_h w[t,h] * max(0, q8[t,h,:] . k8[s,:])
 * for s in 0..p_t; entries with s > p_t are not written.
 *   q_fp8   device uint8 [num_tokens, 64, 128], 16-byte aligned
 *   w       device fp32 [num_tokens, 64] (q_scale etc. already folded in)
 *   logits  device fp32, logits_stride >= max_seq_len
 * Sums are fp32 (fp8 x fp8 products accumulated by the matrix cores).  The
 * kernels evaluate w * max(d, 0) as (w/2) |d| + (w/2) d, the second half
 * through sum_h (w_h/2) q8[t,h,:] held in four fp8 pieces (about 16
 * significant bits; with exact dot products this split rounds to about 1e-7
 * of sum_h |w_h| |d_h| ks).  The dot products come from gfx950's fp8 matrix
 * cores, whose 128-product accumulation is not exact: up to about 2e-4 of
 * sum_d |q_hd k_d| per product, which puts the scores within about 2e-5 of
 * sum_h |w_h| |d_h| ks on N(0,1) data.  A token's scores are the same bits
 * whichever kernel, batch composition or entry point computes them.
 */
idx_status_t idx_logits(const uint8_t* q_fp8, const float* w, int32_t n_heads, int32_t head_dim,
                        idx_kcache_t cache, const idx_batch_t* batch,
                        float* logits, int64_t logits_stride, hipStream_t stream);

/* Workspace bytes idx_topk needs for this batch and k (0 for an empty batch). */
size_t idx_topk_workspace_size(const idx_batch_t* batch, int32_t k);

/*
 * Top-k positions per query token into the persistent buffer ([blog] the
 * buffer-allocation snippet: int32 [max_num_batched_tokens, index_topk]; the
 * op body: entries not produced are -1).
 * Row t considers positions 0..p_t of logits row t and keeps the k largest,
 * ties broken by the lower position, -0.0 equal to +0.0.  The row holds the
 * min(k, p_t + 1) selected positions in ascending order, then -1 up to k.
 *   topk       device int32, row t at topk + t*topk_stride, topk_stride >= k
 *   workspace  device, >= idx_topk_workspace_size(batch, k) bytes, 256-byte aligned
 */
idx_status_t idx_topk(const float* logits, int64_t logits_stride, const idx_batch_t* batch,
                      int32_t k, int32_t* topk, int64_t topk_stride,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes idx_score_topk needs for this batch and k. */
size_t idx_score_topk_workspace_size(const idx_batch_t* batch, int32_t k);

/*
 * idx_logits followed by idx_topk in one call, with the same rows as those
 * two on the same inputs.  Decode batches over long rows (the fused path,
 * below) never write their scores: each work-group keeps its chunk's scores on
 * chip and passes on only the keys above a per-chunk threshold, and one exact
 * select per row takes the top k from them.  Other batches keep the scores in
 * the workspace between the scoring and the select.
 */
idx_status_t idx_score_topk(const uint8_t* q_fp8, const float* w, int32_t n_heads, int32_t head_dim,
                            idx_kcache_t cache, const idx_batch_t* batch, int32_t k,
                            int32_t* topk, int64_t topk_stride,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two launches of idx_score_topk's fused path, for callers that want to
 * run or time them apart.  The fused path serves batches scored one token per
 * work-group (every request has at most one new token, or num_decode_tokens
 * == num_tokens) with fewer than 256 tokens and rows longer than 8192
 * positions; for any other batch both calls return IDX_ERR_UNSUPPORTED.
 * idx_score_candidates scores every causal position with the scores kept on
 * chip and leaves, per chunk of positions, the keys at or above a per-chunk
 * threshold (with the threshold and the chunk's largest key) in the
 * workspace; with k_bf16 != NULL it also quantises this step's new K rows
 * into the cache as idx_quant_write_k would (inside the scoring kernel when
 * every request has at most 4 new tokens).  idx_select_candidates then writes
 * each row's top k exactly as idx_score_topk (rescoring a row whose chunks
 * held more than their share of its top k).  Between the two the workspace,
 * q_fp8, w and the cache must not change.  Workspace: idx_score_topk_workspace_size.
 */
idx_status_t idx_score_candidates(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                  int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                  int32_t k, const uint16_t* k_bf16, int64_t k_row_stride,
                                  const int64_t* slot_mapping, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);
idx_status_t idx_select_candidates(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                   int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                   int32_t k, int32_t* topk, int64_t topk_stride, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);
/* The same two launches over an FP4 cache (the fused path of idx_score_topk_fp4). */
idx_status_t idx_score_candidates_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                      int32_t head_dim, idx_kcache_t cache,
                                      const idx_batch_t* batch, int32_t k, const uint16_t* k_bf16,
                                      int64_t k_row_stride, const int64_t* slot_mapping,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);
idx_status_t idx_select_candidates_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                       int32_t head_dim, idx_kcache_t cache,
                                       const idx_batch_t* batch, int32_t k, int32_t* topk,
                                       int64_t topk_stride, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * The FP4 indexer K cache ([blog] SparseAttnIndexer.forward_cuda passes
 * use_fp4_cache to the op; the pages give no format, the one below is this
 * library's: the OCP MX FP4 element E2M1 with E8M0 power-of-two scales per
 * 32 dims, which gfx950's scaled matrix cores read directly).  Same
 * idx_kcache_t, block_size 64, but each block holds 4352 bytes (68 per
 * position, half the FP8 cache's codes plus four scale bytes):
 *   codes   byte g*1024 + p*16 + i            dims 32g+2i (bits 0-3) and
 *                                             32g+2i+1 (bits 4-7) of offset p
 *   scales  byte 4096 + g*64 + (p%16)*4 + p/16  E8M0 byte e + 127 of group g
 * for groups g = 0..3 of 32 dims and offsets p = 0..63; cache.data holds
 * num_blocks * 4352 bytes, 16-byte aligned.
 *
 * idx_quant_write_k_fp4: per row and group, e = the smallest integer with
 * max(amax_g, 1e-4) <= 6 * 2^e, code = E2M1(x / 2^e) to nearest, ties to
 * even, sign of zero kept; arguments and skipped slots as idx_quant_write_k.
 * Only the written slots' 68 bytes change.
 *
 * idx_logits_fp4: the scores of idx_logits with K decoded group by group,
 *   I[t, s] = sum_h w[t, h] * max(0, sum_d q8[t, h, d] * c[s, d] * 2^e[s, d/32]),
 * same arguments, causal rows and ReLU split (no separate per-position scale).
 *
 * idx_score_topk_fp4: idx_logits_fp4 then idx_topk's selection, with the
 * same rows as those two on the same inputs; decode batches over long rows
 * take the fused path of idx_score_topk (scores kept on chip, per-chunk
 * candidates, one exact select per row), the others keep the scores in the
 * workspace (>= idx_score_topk_fp4_workspace_size bytes, 256-byte aligned).
 */
idx_status_t idx_quant_write_k_fp4(const uint16_t* k_bf16, int64_t num_tokens, int32_t head_dim,
                                   int64_t k_row_stride, const int64_t* slot_mapping,
                                   idx_kcache_t cache, hipStream_t stream);
idx_status_t idx_logits_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads, int32_t head_dim,
                            idx_kcache_t cache, const idx_batch_t* batch, float* logits,
                            int64_t logits_stride, hipStream_t stream);
size_t idx_score_topk_fp4_workspace_size(const idx_batch_t* batch, int32_t k);
idx_status_t idx_score_topk_fp4(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                int32_t k, int32_t* topk, int64_t topk_stride, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * idx_score_topk with its workspace taken from a device array that the
 * library holds, IDX_NOALLOC_SCRATCH_BYTES per device, from the first call
 * on a device until the process ends.  The call itself allocates nothing.
 * It uses the current device's array, so `stream` must belong to the current
 * device.  Results equal idx_score_topk's on the same inputs.
 * Returns IDX_ERR_WORKSPACE when idx_score_topk_workspace_size(batch, k)
 * exceeds IDX_NOALLOC_SCRATCH_BYTES (nothing is launched), and
 * IDX_ERR_LAUNCH if the array's device address cannot be looked up.  Every
 * call on a device shares that device's array, and nothing in it needs to
 * start at zero: calls that overlap on one device (other streams, other
 * threads) race and must be ordered by the caller.
 */
#define IDX_NOALLOC_SCRATCH_BYTES (32u << 20)

idx_status_t idx_score_topk_noalloc(const uint8_t* q_fp8, const float* w, int32_t n_heads,
                                    int32_t head_dim, idx_kcache_t cache, const idx_batch_t* batch,
                                    int32_t k, int32_t* topk, int64_t topk_stride,
                                    hipStream_t stream);

/*
 * IndexCache schedule ([blog] skip_topk snippet; [pr] deepseek_v2.py snippet
 * and Risks & impact).  Host-only.  is_full[l] = 1 for an F layer (runs the
 * indexer, refreshes the top-k buffer), 0 for an S layer (reuses it).
 *   use_index_cache == 0          every layer is F
 *   pattern == NULL               F iff max(l - offset + 1, 0) % freq == 0
 *   pattern != NULL               F iff pattern[l] == 'F'
 * Returns IDX_ERR_INVALID_ARG if freq < 1, num_layers < 1, is_full is NULL,
 * the pattern's length is not num_layers, it holds a character other than
 * 'F' or 'S', or the resulting first layer is S (no producer would have
 * written the buffer before it).
 */
idx_status_t idx_layer_schedule(int32_t use_index_cache, const char* pattern, int32_t freq,
                                int32_t offset, int32_t num_layers, uint8_t* is_full);

/*
 * One indexer layer under IndexCache ([blog] MLA forward: the indexer runs
 * only when the layer does not skip top-k; [pr] mla.py snippet).
 * If is_full or write_k: idx_quant_write_k(layer->k_bf16 ...) into layer->cache.
 * If is_full: idx_score_topk into topk.  An S layer leaves topk untouched, so
 * its consumer reads the rows of the most recent F layer.
 * layer->q_fp8 and layer->w may be NULL on S layers.
 * On an F layer whose batch is scored one token per work-group (every
 * request has one new token, or num_decode_tokens == num_tokens with at most
 * 4 new tokens per request) the new rows are written by the scoring kernel
 * itself, which scores each new row from registers.  The cache bytes and the
 * top-k rows are those of the separate calls whenever every new token's slot
 * is the block-table slot of its position (as the serving metadata has it);
 * a row whose slot differs is still written, but its position is then scored
 * from the cache's previous contents.
 */
typedef struct idx_layer_io {
  const uint16_t* k_bf16;   /* new K rows [num_tokens, k_row_stride] bf16 bits */
  int64_t k_row_stride;
  idx_kcache_t cache;       /* this layer's K cache */
  const uint8_t* q_fp8;     /* [num_tokens, 64, 128] */
  const float* w;           /* [num_tokens, 64] */
} idx_layer_io_t;

idx_status_t idx_indexcache_layer(const idx_layer_io_t* layer, int32_t is_full, int32_t write_k,
                                  const int64_t* slot_mapping, const idx_batch_t* batch, int32_t k,
                                  int32_t* topk, int64_t topk_stride,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * idx_indexcache_layer over an FP4 cache (layer->cache in the FP4 layout
 * described with idx_quant_write_k_fp4): an F layer quantises this step's K
 * rows into it (inside the fused scoring kernel when every request has at
 * most 4 new tokens) and runs idx_score_topk_fp4 (workspace:
 * idx_score_topk_fp4_workspace_size); an S layer writes the K rows (write_k)
 * and nothing else.
 */
idx_status_t idx_indexcache_layer_fp4(const idx_layer_io_t* layer, int32_t is_full,
                                      int32_t write_k, const int64_t* slot_mapping,
                                      const idx_batch_t* batch, int32_t k, int32_t* topk,
                                      int64_t topk_stride, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * A whole stack: idx_indexcache_layer for l = 0..num_layers-1 in order, with
 * is_full from idx_layer_schedule (is_full[0] must be 1) and write_k_on_s
 * choosing whether S layers still write their K rows.
 */
idx_status_t idx_indexcache_stack(const idx_layer_io_t* layers, int32_t num_layers,
                                  const uint8_t* is_full, int32_t write_k_on_s,
                                  const int64_t* slot_mapping, const idx_batch_t* batch, int32_t k,
                                  int32_t* topk, int64_t topk_stride,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The consumer's view of the top-k rows for the logical -> physical
 * conversion ([group] SparseMLAIndexGroup: the physical top-k and the valid
 * counts of an index group): rows are converted through the batch's block
 * table with `block_size` positions per block, physical slot =
 * block * block_stride_rows + offset (block_stride_rows 0 = block_size).
 *   physical      device int32 rows of k entries, physical_stride >= k
 *   valid_counts  device int32 [num_tokens] or NULL
 *   num_blocks    the consumer's pool: a block id outside it gives -1
 */
typedef struct idx_physical {
  int32_t* physical;
  int64_t physical_stride;
  int32_t* valid_counts;
  int32_t block_size;
  int64_t num_blocks;
  int64_t block_stride_rows;
} idx_physical_t;

/*
 * idx_indexcache_layer / idx_indexcache_stack with the group's physical rows
 * ([group] SparseMLAIndexGroup._convert_once, SparseMLAIndexGroupBuilder: a
 * group is the layer that produces the top-k and the layers that reuse it;
 * its rows are converted once, after the producer).  An F layer converts its
 * fresh top-k rows into phys (as idx_topk_to_physical would); an S layer
 * leaves phys alone, so every layer of a group reads the physical rows of the
 * group's F layer.  phys == NULL gives the plain calls.  The physical
 * arguments are checked like idx_topk_to_physical's, before anything is
 * enqueued.
 */
idx_status_t idx_indexcache_layer_physical(const idx_layer_io_t* layer, int32_t is_full,
                                           int32_t write_k, const int64_t* slot_mapping,
                                           const idx_batch_t* batch, int32_t k, int32_t* topk,
                                           int64_t topk_stride, const idx_physical_t* phys,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);
idx_status_t idx_indexcache_stack_physical(const idx_layer_io_t* layers, int32_t num_layers,
                                           const uint8_t* is_full, int32_t write_k_on_s,
                                           const int64_t* slot_mapping, const idx_batch_t* batch,
                                           int32_t k, int32_t* topk, int64_t topk_stride,
                                           const idx_physical_t* phys, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/*
 * Logical -> physical top-k conversion ([group] SparseMLAIndexGroup,
 * convert_logical_to_physical_topk / _convert_once): for token t of request
 * r, physical = block_table[r][pos / block_size] * stride_rows + pos % block_size,
 * -1 stays -1; valid_counts[t] = number of entries >= 0 in row t.
 *   logical, physical   device int32 rows of k entries (strides >= k)
 *   block_stride_rows   rows per physical block (0 = block_size)
 *   valid_counts        device int32 [num_tokens] or NULL
 * A logical position outside 0..p_t (or a block id outside the pool) gives -1.
 */
idx_status_t idx_topk_to_physical(const int32_t* logical, int64_t logical_stride,
                                  const idx_batch_t* batch, int32_t block_size, int64_t num_blocks,
                                  int32_t k, int64_t block_stride_rows,
                                  int32_t* physical, int64_t physical_stride,
                                  int32_t* valid_counts, hipStream_t stream);

/*
 * Per-kernel timing without a profiler (diagnostics; not part of the method).
 * After idx_trace_begin(events, capacity), every kernel the library enqueues
 * from the calling thread is bracketed by two of the caller's events:
 * events[2i] is recorded on the kernel's stream just before kernel i and
 * events[2i+1] just after it, until the events run out (later kernels are not
 * bracketed).  idx_trace_end stops the trace and returns the number of kernels
 * bracketed; with names != NULL, names[i] (static strings, i < max_names)
 * receives kernel i's name.  The events belong to the caller (created with
 * timing enabled).  Recording events adds work to the stream, so a traced call
 * runs slightly slower than an untraced one, and a trace under graph capture
 * records event nodes into the graph.  idx_trace_begin returns
 * IDX_ERR_INVALID_ARG for a null array or a capacity below 2.
 */
idx_status_t idx_trace_begin(hipEvent_t* events, int32_t capacity);
int32_t idx_trace_end(const char** names, int32_t max_names);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H_ */

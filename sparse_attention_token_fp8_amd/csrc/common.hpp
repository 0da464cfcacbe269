// Internal definitions shared by the libidx sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "idx.h"

namespace idx {

constexpr int kHeadDim = 128;                   // indexer head_dim (the blog's Indexer.__init__)
constexpr int kHeads = 64;                      // indexer query heads
constexpr int kBlock = 64;                      // paged block_size
constexpr int kTokenBytes = kHeadDim + 4;       // 128 code bytes + fp32 scale
constexpr int kBlockBytes = kBlock * kTokenBytes;  // 8448
constexpr int kCodeBytes = kBlock * kHeadDim;      // 8192: the scales follow the codes
constexpr int kMaxK = 2048;

// Top-k radix digits: bits [31:21] of the order key (level 1, also the
// histogram the scoring kernels build), then [20:10], then [9:0].
constexpr int kBins1 = 2048;
constexpr int kShift1 = 21;
constexpr int kBins2 = 2048;
constexpr int kShift2 = 10;
constexpr int kBins3 = 1024;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Batch metadata as the kernels take it (by value).
struct BatchArgs {
  const int32_t* seq_lens;
  const int32_t* qsl;
  const int32_t* bt;
  int64_t bt_stride;
  int32_t num_reqs;
  int32_t num_tokens;
  int32_t max_seq_len;
  int32_t max_query_len;
};

struct CacheArgs {
  const uint8_t* data;
  int64_t num_blocks;
};

// Per-row top-k bookkeeping in the workspace (64 bytes per row).
struct RowState {
  uint32_t done_hist;    // producer work-groups finished (histogram complete when == chunks)
  uint32_t done_filter;  // filter work-groups finished
  uint32_t b1;           // level-1 threshold digit
  uint32_t need;         // k - #(digit > b1)
  uint32_t n_above;      // append counter of the above list
  uint32_t n_cand;       // append counter of the candidate list
  uint32_t cand_total;   // hist[b1]
  uint32_t pad[9];
};

// Workspace carve-up shared by the host sizing code and the launchers.
struct TopkWorkspace {
  RowState* state;     // [T]
  uint32_t* hist;      // [T][kBins1]
  int32_t* above;      // [T][k]
  uint32_t* cand;      // [T][cap][2] (key, position)
  float* logits;       // [T][ld] (fused path only)
  int64_t ld;
  int32_t cap;
  int32_t k;
};

constexpr int kCandCap = 4096;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout of a top-k workspace for T rows; returns total bytes.  When base is
// non-null also fills `ws`.
inline size_t topk_workspace_layout(int64_t T, int32_t k, int64_t logits_ld, void* base,
                                    TopkWorkspace* ws) {
  size_t off = 0;
  const size_t o_state = off;  off = align_up(off + sizeof(RowState) * (size_t)T, 256);
  const size_t o_hist = off;   off = align_up(off + sizeof(uint32_t) * kBins1 * (size_t)T, 256);
  const size_t o_above = off;  off = align_up(off + sizeof(int32_t) * (size_t)k * (size_t)T, 256);
  const size_t o_cand = off;   off = align_up(off + 2 * sizeof(uint32_t) * kCandCap * (size_t)T, 256);
  const size_t o_logits = off; off = align_up(off + sizeof(float) * (size_t)logits_ld * (size_t)T, 256);
  if (base && ws) {
    char* b = static_cast<char*>(base);
    ws->state = reinterpret_cast<RowState*>(b + o_state);
    ws->hist = reinterpret_cast<uint32_t*>(b + o_hist);
    ws->above = reinterpret_cast<int32_t*>(b + o_above);
    ws->cand = reinterpret_cast<uint32_t*>(b + o_cand);
    ws->logits = logits_ld ? reinterpret_cast<float*>(b + o_logits) : nullptr;
    ws->ld = logits_ld;
    ws->cap = kCandCap;
    ws->k = k;
  }
  return off;
}

// Bytes the per-call clear must zero (state + histograms).
inline size_t topk_workspace_clear_bytes(int64_t T) {
  return align_up(sizeof(RowState) * (size_t)T, 256) + sizeof(uint32_t) * kBins1 * (size_t)T;
}

// ---------------------------------------------------------------- device --

// Monotone map float -> uint32 (larger float, larger key); -0 maps to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Request of query token t: the largest r with qsl[r] <= t (bounded search).
__device__ __forceinline__ int find_request(const int32_t* __restrict__ qsl, int num_reqs, int t) {
  int lo = 0, hi = num_reqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct TokenPos {
  int r;  // request
  int n;  // number of causal positions (p_t + 1), clamped to [0, max_seq_len]
};

__device__ __forceinline__ TokenPos token_pos(const BatchArgs& b, int t) {
  TokenPos tp;
  tp.r = find_request(b.qsl, b.num_reqs, t);
  const int q0 = b.qsl[tp.r];
  const int nr = b.qsl[tp.r + 1] - q0;
  int n = b.seq_lens[tp.r] - nr + (t - q0) + 1;
  n = n < 0 ? 0 : n;
  tp.n = n > b.max_seq_len ? b.max_seq_len : n;
  return tp;
}

// Physical block of logical block `lb` of request r, or -1 if it lies outside
// the block table or the pool.
__device__ __forceinline__ int64_t phys_block(const BatchArgs& b, const CacheArgs& c, int r, int lb) {
  if (lb < 0 || lb >= b.bt_stride) return -1;
  const int64_t blk = b.bt[(int64_t)r * b.bt_stride + lb];
  return (blk >= 0 && blk < c.num_blocks) ? blk : -1;
}

// Agent-scope loads of values other work-groups updated with atomics.
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace idx

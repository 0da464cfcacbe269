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

// Top-k radix digits of the order key: bits [31:21], then [20:10], then [9:0].
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

// Sample of a row used to place the top-k threshold: positions
// j*S + ((37*j + 11) & (S-1)), S a power of two chosen so that at most
// kMaxSample positions are drawn.
constexpr int kMaxSample = 2048;

__host__ __device__ inline int sample_stride(int n) {
  int S = 16;
  while ((n + S - 1) / S > kMaxSample) S <<= 1;
  return S;
}

__host__ __device__ inline int sample_pos(int j, int S) { return j * S + ((37 * j + 11) & (S - 1)); }

// Top-k workspace (device, caller-owned).  The fused entry points keep the
// scores in `logits` and, for every row long enough to be sampled, the row's
// sampled scores in `samp` (entry j = the score at sample_pos(j, S)), written
// by the scoring kernels.
// Long rows keep their candidates in `nslots` slots of `slot_cap` entries per
// row (`cand_key` / `cand_pos`, in position order across the slots; one slot
// per chunk of topk_chunk() positions) with each slot's count in `counts`.
struct TopkWorkspace {
  float* logits;       // [T][ld] (fused path only)
  float* samp;         // [T][kMaxSample] (fused path, long rows only)
  uint32_t* cand_key;  // [T][nslots][slot_cap]
  int32_t* cand_pos;   // [T][nslots][slot_cap]
  uint32_t* counts;    // [T][nslots]
  int64_t ld;
  int32_t nslots;
  int32_t slot_cap;
};

// Workspace of the fused score + top-k for decode-split batches over long
// rows: each (row, chunk) slot holds up to `cap` candidates (key, position) in
// position order, their count, the chunk's threshold and its largest key.  cap
// is the chunk's positions (chunk_blocks * 64), so a row's slots can also hold
// all its keys as one flat array when the row has to be rescored.
struct KeepSlots {
  uint2* cand;         // [T][nslots][cap] (key, position)
  uint32_t* counts;    // [T][nslots]
  uint32_t* taus;      // [T][nslots]
  uint32_t* maxes;     // [T][nslots]: the chunk's largest key
  int32_t nslots;
  int32_t cap;
  int32_t chunk_blocks;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool topk_uses_long_rows(int64_t T, int max_seq_len);
// Filter chunk (positions per slot); shorter when the sample copy exists.
int topk_chunk(bool sample_copy);
int topk_nchunks(int max_seq_len, bool sample_copy);
int topk_max_seq_len();

constexpr int kMaxSlots = 2048;                 // slots per row the resolve can index
constexpr int kRowCap = 5120;                   // LDS candidates of the many-rows top-k; longer rows are sampled

// Layout of the workspace for T rows of up to max_seq_len positions; returns
// the total bytes.  When base is non-null also fills `ws`.  logits_ld is 0
// for idx_topk (scores come from the caller).
inline size_t topk_workspace_layout(int64_t T, int max_seq_len, int64_t logits_ld, void* base,
                                    TopkWorkspace* ws) {
  const bool lr = topk_uses_long_rows(T, max_seq_len);
  // the scoring kernels' compact sample copy, for every row a tau is sampled for
  const bool samp = logits_ld > 0 && (lr || max_seq_len > kRowCap);
  const int64_t nslots = lr ? topk_nchunks(max_seq_len, samp) : 0;
  const int64_t cap = lr ? topk_chunk(samp) : 0;
  size_t off = 0;
  const size_t o_logits = off;
  off = align_up(off + sizeof(float) * (size_t)logits_ld * (size_t)T, 256);
  const size_t o_ckey = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)cap * (size_t)nslots * (size_t)T, 256);
  const size_t o_cpos = off;
  off = align_up(off + sizeof(int32_t) * (size_t)cap * (size_t)nslots * (size_t)T, 256);
  const size_t o_counts = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)nslots * (size_t)T, 256);
  const size_t o_samp = off;
  off = align_up(off + (samp ? sizeof(float) * (size_t)kMaxSample * (size_t)T : 0), 256);
  if (off == 0) off = 256;
  if (base && ws) {
    char* b = static_cast<char*>(base);
    ws->logits = logits_ld ? reinterpret_cast<float*>(b + o_logits) : nullptr;
    ws->samp = samp ? reinterpret_cast<float*>(b + o_samp) : nullptr;
    ws->cand_key = reinterpret_cast<uint32_t*>(b + o_ckey);
    ws->cand_pos = reinterpret_cast<int32_t*>(b + o_cpos);
    ws->counts = reinterpret_cast<uint32_t*>(b + o_counts);
    ws->ld = logits_ld;
    ws->nslots = (int32_t)nslots;
    ws->slot_cap = (int32_t)cap;
  }
  return off;
}

// ---------------------------------------------------------------- device --

// ------------------------------------------------------ wave primitives --
// Scans and reductions over the 64 lanes of a wave with DPP moves (row shifts
// within rows of 16 lanes, then row broadcasts): a few cycles per step, where
// a lane shuffle is a round trip through the LDS.  Every lane must be active.
// `id` is the operation's identity; lanes with no source lane receive it.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// Inclusive prefix sum over the lanes (lane i: v_0 + ... + v_i).
__device__ __forceinline__ uint32_t wave_sum_incl(uint32_t v) {
  return wave_scan_incl(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// The sum / max / min over the wave, in every lane (a wave-uniform value).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_sum_incl(v), 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane(
      (int)wave_scan_incl(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }), 63);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane(
      (int)wave_scan_incl(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; }), 63);
}

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
  int r;    // request
  int n;    // number of causal positions (p_t + 1), clamped to [0, max_seq_len]
  int q0;   // the request's first query token
  int nq;   // the request's number of new tokens
  int len;  // the request's sequence length
};

__device__ __forceinline__ TokenPos token_pos(const BatchArgs& b, int t) {
  TokenPos tp;
  tp.r = find_request(b.qsl, b.num_reqs, t);
  tp.q0 = b.qsl[tp.r];
  tp.nq = b.qsl[tp.r + 1] - tp.q0;
  tp.len = b.seq_lens[tp.r];
  int n = tp.len - tp.nq + (t - tp.q0) + 1;
  n = n < 0 ? 0 : n;
  tp.n = n > b.max_seq_len ? b.max_seq_len : n;
  return tp;
}

// token_pos for a whole wave (every lane active, same t): with fewer than 256
// requests the lanes read query_start_loc and seq_lens in one round (request
// 64u + lane in slot u) and ballots find the request, so the lookup costs one
// load latency, not a search.
__device__ __forceinline__ TokenPos token_pos_wave(const BatchArgs& b, int t) {
  constexpr int U = 4;
  if (b.num_reqs >= 64 * U) return token_pos(b, t);
  const int lane = threadIdx.x & 63;
  int q[U], len[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = 64 * u + lane;
    q[u] = r <= b.num_reqs ? b.qsl[r] : 0x7fffffff;
    len[u] = r < b.num_reqs ? b.seq_lens[r] : 0;
  }
  int m = 0;                                    // requests starting at or before t
#pragma unroll
  for (int u = 0; u < U; ++u)
    m += (int)__popcll(__ballot(64 * u + lane < b.num_reqs && q[u] <= t));
  TokenPos tp;
  tp.r = m > 0 ? m - 1 : 0;
  // the value of request r (uniform) from its slot; values, not the arrays,
  // are passed so that q[] and len[] stay in registers
  auto pick = [](int v0, int v1, int v2, int v3, int r) {
    const int u = r >> 6;
    const int x = u == 0 ? v0 : u == 1 ? v1 : u == 2 ? v2 : v3;
    return __builtin_amdgcn_readlane(x, r & 63);
  };
  static_assert(U == 4, "pick takes four slots");
  tp.q0 = pick(q[0], q[1], q[2], q[3], tp.r);
  tp.nq = pick(q[0], q[1], q[2], q[3], tp.r + 1) - tp.q0;
  tp.len = pick(len[0], len[1], len[2], len[3], tp.r);
  int n = tp.len - tp.nq + (t - tp.q0) + 1;
  n = n < 0 ? 0 : n;
  tp.n = n > b.max_seq_len ? b.max_seq_len : n;
  return tp;
}

// A buffer resource over the `bytes` bytes at `base` (gfx9 raw buffer, data
// format 32).  A load from an offset at or past `bytes` returns zeros and
// moves no data: the hardware's range check, which the staging loops use for
// blocks that are absent or past the end, so that every load stays
// unconditional without fetching anything.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Buffer-load cache policy: non-temporal (streamed past the caches).
constexpr int kLoadStream = 2;

// Physical block of logical block `lb` of request r, or -1 if it lies outside
// the block table or the pool.
__device__ __forceinline__ int64_t phys_block(const BatchArgs& b, const CacheArgs& c, int r, int lb) {
  if (lb < 0 || lb >= b.bt_stride) return -1;
  const int64_t blk = b.bt[(int64_t)r * b.bt_stride + lb];
  return (blk >= 0 && blk < c.num_blocks) ? blk : -1;
}

}  // namespace idx

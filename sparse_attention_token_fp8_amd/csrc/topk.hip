// Radix top-k select over the causal scores of each query token.
//
// Pages: IndexCache blog post -- the persistent topk_indices_buffer is int32
// [max_num_batched_tokens, index_topk] and entries not produced hold -1 (the op
// body and the buffer-allocation snippet).  Selection rule: the k largest
// scores of positions 0..p_t, ties to the lower position, -0 == +0; a row lists
// the selected positions in ascending order, then -1.
//
// Scores map to order-preserving 32-bit keys.  Digits are bits [31:21],
// [20:10], [9:0].
//   1. level-1 histogram of the row (here, or fused into the decode scoring
//      kernel); the last work-group of the row picks b1, the digit that holds
//      the k-th largest key;
//   2. filter: every key with digit > b1 is selected outright (fewer than k of
//      them); keys with digit == b1 become candidates (key, position);
//   3. the last filter work-group of the row resolves the candidates with two
//      more LDS histograms to the exact k-th key K* and the number of keys equal
//      to K* still to take (lowest positions first), then writes the row in
//      ascending position order through an LDS bitmap, segment by segment.
// When a row's candidate bin is larger than the workspace list, step 3 reads
// the row itself instead of the list.

#include "common.hpp"
#include "launch.hpp"
#include "topk_device.hpp"

namespace idx {
namespace {

constexpr int kChunk = 4096;               // positions per work-group in hist / filter
constexpr int kPerThread = kChunk / kThreads;
constexpr int kSeg = 65536;                // positions per bitmap segment in the resolve
constexpr int kSegWords = kSeg / 32;
constexpr int kWordsPerThread = kSegWords / kThreads;

__global__ __launch_bounds__(256) void clear_kernel(uint4* __restrict__ p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(256) void hist_kernel(const float* __restrict__ logits, int64_t ld,
                                                   BatchArgs b, TopkWorkspace ws, int k) {
  const int t = blockIdx.y;
  const int n = token_pos(b, t).n;
  if (n <= k) return;
  const int s0 = blockIdx.x * kChunk;
  if (s0 >= n) return;
  __shared__ uint32_t lhist[kBins1];
  __shared__ uint32_t scratch[8];
  for (int i = threadIdx.x; i < kBins1; i += kThreads) lhist[i] = 0;
  __syncthreads();
  const float* row = logits + (size_t)t * ld;
#pragma unroll 4
  for (int i = 0; i < kPerThread; ++i) {
    const int s = s0 + threadIdx.x + i * kThreads;
    if (s < n) atomicAdd(&lhist[order_key(row[s]) >> kShift1], 1u);
  }
  finish_hist(ws, t, k, (n + kChunk - 1) / kChunk, lhist, scratch);
}

// Visit the candidates of row t (digit == b1): from the list, or from the row.
template <typename F>
__device__ __forceinline__ void for_each_candidate(const TopkWorkspace& ws, const float* row, int n,
                                                   int t, uint32_t b1, bool use_list,
                                                   uint32_t n_list, F&& fn) {
  if (use_list) {
    const uint32_t* cl = ws.cand + (size_t)t * ws.cap * 2;
    for (uint32_t i = threadIdx.x; i < n_list; i += kThreads) fn(cl[2 * i], (int)cl[2 * i + 1]);
  } else {
    for (int s = threadIdx.x; s < n; s += kThreads) {
      const uint32_t key = order_key(row[s]);
      if ((key >> kShift1) == b1) fn(key, s);
    }
  }
}

// Find the digit d (0..nb-1, searched from the top) with
// #(digit > d) < need <= #(digit >= d) in an LDS histogram; returns d and
// sets *above = #(digit > d).  All threads get the result.
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, int nb, uint32_t need,
                                               uint32_t* above, uint32_t* scratch) {
  const int per = nb / kThreads;  // 8 or 4
  const int top = nb - 1 - per * (int)threadIdx.x;
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) sum += h[top - j];
  uint32_t total;
  const uint32_t before = block_exclusive_scan(sum, &total, scratch);
  if (before < need && before + sum >= need) {
    uint32_t cum = before;
    for (int j = 0; j < per; ++j) {
      const uint32_t c = h[top - j];
      if (cum + c >= need) {
        scratch[5] = (uint32_t)(top - j);
        scratch[6] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  const uint32_t d = scratch[5];
  *above = scratch[6];
  __syncthreads();
  return d;
}

__device__ void resolve_row(const TopkWorkspace& ws, const float* row, int n, int t, int k,
                            int32_t* out, uint32_t* lds, uint32_t* scratch) {
  RowState* st = ws.state + t;
  const uint32_t b1 = st->b1;
  const uint32_t n_above = min(load_agent(&st->n_above), (uint32_t)k);
  const uint32_t cand_total = st->cand_total;
  const bool use_list = cand_total <= (uint32_t)ws.cap;
  const uint32_t n_list = use_list ? min(load_agent(&st->n_cand), (uint32_t)ws.cap) : 0u;
  const uint32_t need = (uint32_t)k - n_above;   // >= 1

  // level 2: digit [20:10] among the candidates
  for (int i = threadIdx.x; i < kBins2; i += kThreads) lds[i] = 0;
  __syncthreads();
  for_each_candidate(ws, row, n, t, b1, use_list, n_list, [&](uint32_t key, int) {
    atomicAdd(&lds[(key >> kShift2) & (kBins2 - 1)], 1u);
  });
  __syncthreads();
  uint32_t above2;
  const uint32_t b2 = find_digit(lds, kBins2, need, &above2, scratch);
  const uint32_t need2 = need - above2;

  // level 3: digit [9:0] among candidates with digits (b1, b2)
  for (int i = threadIdx.x; i < kBins3; i += kThreads) lds[i] = 0;
  __syncthreads();
  for_each_candidate(ws, row, n, t, b1, use_list, n_list, [&](uint32_t key, int) {
    if (((key >> kShift2) & (kBins2 - 1)) == b2) atomicAdd(&lds[key & (kBins3 - 1)], 1u);
  });
  __syncthreads();
  uint32_t above3;
  const uint32_t b3 = find_digit(lds, kBins3, need2, &above3, scratch);
  const uint32_t take_eq = need2 - above3;        // keys equal to K* to take, lowest positions first
  const uint32_t kstar = (b1 << kShift1) | (b2 << kShift2) | b3;

  // emit in ascending position order, one bitmap segment at a time
  uint32_t* sel = lds;
  uint32_t* tie = lds + kSegWords;
  const int32_t* al = ws.above + (size_t)t * k;
  uint32_t written = 0, ties_taken = 0;
  for (int g0 = 0; g0 < n; g0 += kSeg) {
    for (int i = threadIdx.x; i < 2 * kSegWords; i += kThreads) lds[i] = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_above; i += kThreads) {
      const int s = al[i] - g0;
      if (s >= 0 && s < kSeg) atomicOr(&sel[s >> 5], 1u << (s & 31));
    }
    for_each_candidate(ws, row, n, t, b1, use_list, n_list, [&](uint32_t key, int pos) {
      const int s = pos - g0;
      if (s < 0 || s >= kSeg) return;
      if (key > kstar) atomicOr(&sel[s >> 5], 1u << (s & 31));
      else if (key == kstar) atomicOr(&tie[s >> 5], 1u << (s & 31));
    });
    __syncthreads();
    // ties: keep the first (take_eq - ties_taken) of this segment, in order
    const int w0 = threadIdx.x * kWordsPerThread;
    uint32_t my_ties = 0;
    for (int j = 0; j < kWordsPerThread; ++j) my_ties += __popc(tie[w0 + j]);
    uint32_t seg_ties;
    uint32_t tie_before = ties_taken + block_exclusive_scan(my_ties, &seg_ties, scratch);
    for (int j = 0; j < kWordsPerThread; ++j) {
      uint32_t word = tie[w0 + j];
      while (word) {
        const uint32_t bit = word & (0u - word);
        word ^= bit;
        if (tie_before < take_eq) sel[w0 + j] |= bit;
        ++tie_before;
      }
    }
    ties_taken += seg_ties;
    __syncthreads();
    uint32_t my_sel = 0;
    for (int j = 0; j < kWordsPerThread; ++j) my_sel += __popc(sel[w0 + j]);
    uint32_t seg_sel;
    uint32_t o = written + block_exclusive_scan(my_sel, &seg_sel, scratch);
    for (int j = 0; j < kWordsPerThread; ++j) {
      uint32_t word = sel[w0 + j];
      while (word) {
        const int bitpos = __ffs(word) - 1;
        word &= word - 1;
        if (o < (uint32_t)k) out[o] = g0 + (w0 + j) * 32 + bitpos;
        ++o;
      }
    }
    written += seg_sel;
    __syncthreads();
  }
  for (uint32_t i = written + threadIdx.x; i < (uint32_t)k; i += kThreads) out[i] = -1;
}

__global__ __launch_bounds__(256) void filter_kernel(const float* __restrict__ logits, int64_t ld,
                                                     BatchArgs b, TopkWorkspace ws, int k,
                                                     int32_t* __restrict__ topk, int64_t ldo) {
  const int t = blockIdx.y;
  const int n = token_pos(b, t).n;
  int32_t* out = topk + (size_t)t * ldo;
  if (n <= k) {  // every causal position is selected
    if (blockIdx.x == 0)
      for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const int s0 = blockIdx.x * kChunk;
  if (s0 >= n) return;
  __shared__ uint32_t lds[2 * kSegWords];
  __shared__ uint32_t scratch[8];
  const float* row = logits + (size_t)t * ld;
  RowState* st = ws.state + t;
  const uint32_t b1 = st->b1;
  const bool use_list = st->cand_total <= (uint32_t)ws.cap;

  uint32_t keys[kPerThread];
  uint32_t na = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int s = s0 + threadIdx.x + i * kThreads;
    uint32_t key = 0;
    if (s < n) {
      key = order_key(row[s]);
      const uint32_t d = key >> kShift1;
      na += d > b1;
      nc += (d == b1 && use_list);
    }
    keys[i] = key;
  }
  uint32_t tot;
  const uint32_t pre = block_exclusive_scan(na | (nc << 16), &tot, scratch);
  if (threadIdx.x == 0) {
    scratch[4] = (tot & 0xFFFF) ? atomicAdd(&st->n_above, tot & 0xFFFF) : 0u;
    scratch[5] = (tot >> 16) ? atomicAdd(&st->n_cand, tot >> 16) : 0u;
  }
  __syncthreads();
  uint32_t ia = scratch[4] + (pre & 0xFFFF);
  uint32_t ic = scratch[5] + (pre >> 16);
  int32_t* al = ws.above + (size_t)t * k;
  uint32_t* cl = ws.cand + (size_t)t * ws.cap * 2;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int s = s0 + threadIdx.x + i * kThreads;
    if (s >= n) continue;
    const uint32_t d = keys[i] >> kShift1;
    if (d > b1) {
      if (ia < (uint32_t)k) al[ia] = s;
      ++ia;
    } else if (d == b1 && use_list) {
      if (ic < (uint32_t)ws.cap) { cl[2 * ic] = keys[i]; cl[2 * ic + 1] = (uint32_t)s; }
      ++ic;
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t chunks = (uint32_t)((n + kChunk - 1) / kChunk);
    scratch[7] = (atomicAdd(&st->done_filter, 1u) == chunks - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (scratch[7]) {
    __threadfence();
    resolve_row(ws, row, n, t, k, out, lds, scratch);
  }
}

}  // namespace

hipError_t launch_topk_clear(const TopkWorkspace& ws, int64_t T, hipStream_t stream) {
  const int64_t n16 = (int64_t)(topk_workspace_clear_bytes(T) / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(ws.state), n16);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* logits, int64_t ld, const BatchArgs& b,
                            const TopkWorkspace& ws, int k, hipStream_t stream) {
  if (b.num_tokens == 0 || b.max_seq_len <= k) return hipSuccess;
  const dim3 grid((unsigned)((b.max_seq_len + kChunk - 1) / kChunk), (unsigned)b.num_tokens);
  hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, stream, logits, ld, b, ws, k);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const float* logits, int64_t ld, const BatchArgs& b,
                              const TopkWorkspace& ws, int k, int32_t* out, int64_t ldo,
                              hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  const int chunks = std::max(1, (b.max_seq_len + kChunk - 1) / kChunk);
  const dim3 grid((unsigned)chunks, (unsigned)b.num_tokens);
  hipLaunchKernelGGL(filter_kernel, grid, dim3(256), 0, stream, logits, ld, b, ws, k, out, ldo);
  return hipGetLastError();
}

}  // namespace idx

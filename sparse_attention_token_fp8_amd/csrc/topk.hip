// Top-k select over the causal scores of each query token (see
// topk_device.hpp for the rule and the method).  Two launch shapes:
//
//   many rows    one 1024-thread work-group per row: tau from the row's sample,
//                candidates (key >= tau) compacted into LDS, exact select,
//                ordered write-out.  No global scratch, no atomics outside LDS.
//   few long rows  filter: work-groups of 4096 positions compact their
//                candidates into a private slot of the workspace (no atomics,
//                nothing to clear); resolve: one work-group per row gathers
//                the slots and finishes as above.
//
// Neither shape uses device-scope atomics or fences: work-groups meet only at
// kernel boundaries.

#include "common.hpp"
#include "launch.hpp"
#include "topk_device.hpp"

namespace idx {
namespace {

constexpr int kRowThreads = 1024;
constexpr int kCandCap = 8192;       // LDS candidate capacity per row
constexpr int kBatch = 8;            // loads in flight per thread in the row kernel

// Trivial rows (p_t + 1 <= k): every position, then -1.
template <int NT>
__device__ __forceinline__ void write_all(int32_t* out, int n, int k) {
  for (int j = threadIdx.x; j < k; j += NT) out[j] = j < n ? j : -1;
}

// Append (key, pos) to an LDS candidate list with one LDS atomic per wave.
__device__ __forceinline__ void append_wave(bool p, uint32_t key, int pos, uint32_t* count,
                                            uint32_t* ckey, int32_t* cpos, uint32_t cap) {
  const int lane = threadIdx.x & 63;
  const uint64_t m = __ballot(p);
  uint32_t base = 0;
  if (lane == 0 && m) base = atomicAdd(count, (uint32_t)__popcll(m));
  base = (uint32_t)__shfl((int)base, 0);
  if (p) {
    const uint32_t slot = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (slot < cap) { ckey[slot] = key; cpos[slot] = pos; }
  }
}

// Exact select over the candidates held in LDS (k <= C <= kCandCap), else over
// the whole row, then the ordered write-out.
template <int NT>
__device__ __forceinline__ void finish_row(const float* __restrict__ row, int n, int k, uint32_t C,
                                           const uint32_t* ckey, const int32_t* cpos,
                                           int32_t* __restrict__ out, uint32_t* work,
                                           uint32_t* scratch) {
  uint32_t take;
  if (C >= (uint32_t)k && C <= (uint32_t)kCandCap) {
    auto visit = [&](auto&& fn) {
      for (uint32_t i = threadIdx.x; i < C; i += NT) fn(ckey[i], cpos[i]);
    };
    const uint32_t kstar = radix_kth<NT>(visit, (uint32_t)k, &take, work, scratch);
    emit_row<NT>(visit, n, kstar, take, k, out, work, scratch);
  } else {
    auto visit = [&](auto&& fn) {
      for (int s = threadIdx.x; s < n; s += NT) fn(order_key(row[s]), s);
    };
    const uint32_t kstar = radix_kth<NT>(visit, (uint32_t)k, &take, work, scratch);
    emit_row<NT>(visit, n, kstar, take, k, out, work, scratch);
  }
}

__global__ __launch_bounds__(kRowThreads) void topk_rows_kernel(const float* __restrict__ logits,
                                                                int64_t ld, BatchArgs b, int k,
                                                                int32_t* __restrict__ topk,
                                                                int64_t ldo) {
  const int t = blockIdx.x;
  const int n = token_pos(b, t).n;
  int32_t* out = topk + (size_t)t * ldo;
  if (n <= k) {
    write_all<kRowThreads>(out, n, k);
    return;
  }
  __shared__ uint32_t ckey[kCandCap];
  __shared__ int32_t cpos[kCandCap];
  __shared__ uint32_t work[2 * kSegWords];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t count;
  const float* row = logits + (size_t)t * ld;
  const uint32_t tau = row_tau<kRowThreads>(row, n, k, kCandCap, work, scratch);
  if (threadIdx.x == 0) count = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kRowThreads * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int s = base + threadIdx.x + e * kRowThreads;
      v[e] = s < n ? row[s] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int s = base + threadIdx.x + e * kRowThreads;
      const uint32_t key = order_key(v[e]);
      append_wave(s < n && key >= tau, key, s, &count, ckey, cpos, kCandCap);
    }
  }
  __syncthreads();
  finish_row<kRowThreads>(row, n, k, count, ckey, cpos, out, work, scratch);
}

// ---------------------------------------------------------- long rows --
constexpr int kChunk = 4096;          // positions per filter work-group
constexpr int kPer = kChunk / kThreads;

__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float* __restrict__ logits,
                                                               int64_t ld, BatchArgs b, int k,
                                                               TopkWorkspace ws,
                                                               int32_t* __restrict__ topk,
                                                               int64_t ldo) {
  const int t = blockIdx.y;
  const int c = blockIdx.x;
  const int n = token_pos(b, t).n;
  if (n <= k) {
    if (c == 0) write_all<kThreads>(topk + (size_t)t * ldo, n, k);
    return;
  }
  const int s0 = c * kChunk;
  if (s0 >= n) return;
  __shared__ uint32_t work[kBins1];
  __shared__ uint32_t scratch[16];
  __shared__ uint32_t count;
  const float* row = logits + (size_t)t * ld;
  const uint32_t tau = row_tau<kThreads>(row, n, k, 4 * k, work, scratch);
  if (threadIdx.x == 0) count = 0;
  __syncthreads();
  uint32_t* slot = ws.cand + ((size_t)t * ws.nchunks + c) * kChunk * 2;
  float v[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int s = s0 + threadIdx.x + e * kThreads;
    v[e] = s < n ? row[s] : 0.f;
  }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int s = s0 + threadIdx.x + e * kThreads;
    const uint32_t key = order_key(v[e]);
    const bool p = s < n && key >= tau;
    const uint64_t m = __ballot(p);
    uint32_t base = 0;
    if (lane == 0 && m) base = atomicAdd(&count, (uint32_t)__popcll(m));
    base = (uint32_t)__shfl((int)base, 0);
    if (p) {
      const uint32_t i = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      slot[2 * i] = key;
      slot[2 * i + 1] = (uint32_t)s;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) ws.counts[(size_t)t * ws.nchunks + c] = count;
}

__global__ __launch_bounds__(kRowThreads) void topk_resolve_kernel(const float* __restrict__ logits,
                                                                   int64_t ld, BatchArgs b, int k,
                                                                   TopkWorkspace ws,
                                                                   int32_t* __restrict__ topk,
                                                                   int64_t ldo) {
  const int t = blockIdx.x;
  const int n = token_pos(b, t).n;
  if (n <= k) return;                          // written by the filter
  __shared__ uint32_t ckey[kCandCap];
  __shared__ int32_t cpos[kCandCap];
  __shared__ uint32_t work[2 * kSegWords];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t count;
  const int nch = (n + kChunk - 1) / kChunk;
  const uint32_t* cnts = ws.counts + (size_t)t * ws.nchunks;
  uint32_t C = 0;
  for (int c = 0; c < nch; ++c) C += cnts[c];
  const float* row = logits + (size_t)t * ld;
  int32_t* out = topk + (size_t)t * ldo;
  if (C >= (uint32_t)k && C <= (uint32_t)kCandCap) {
    // gather the chunk slots into LDS
    uint32_t off = 0;
    for (int c = 0; c < nch; ++c) {
      const uint32_t cn = cnts[c];
      const uint32_t* slot = ws.cand + ((size_t)t * ws.nchunks + c) * kChunk * 2;
      for (uint32_t i = threadIdx.x; i < cn; i += kRowThreads) {
        ckey[off + i] = slot[2 * i];
        cpos[off + i] = (int32_t)slot[2 * i + 1];
      }
      off += cn;
    }
    __syncthreads();
  }
  (void)count;
  finish_row<kRowThreads>(row, n, k, C, ckey, cpos, out, work, scratch);
}

}  // namespace

bool topk_uses_long_rows(int64_t T, int max_seq_len) { return T < 256 && max_seq_len > 8192; }

int topk_nchunks(int max_seq_len) { return (max_seq_len + kChunk - 1) / kChunk; }

int topk_chunk() { return kChunk; }

hipError_t launch_topk(const float* logits, int64_t ld, const BatchArgs& b, const TopkWorkspace& ws,
                       int k, int32_t* out, int64_t ldo, hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  if (topk_uses_long_rows(b.num_tokens, b.max_seq_len)) {
    const dim3 grid((unsigned)std::max(1, topk_nchunks(b.max_seq_len)), (unsigned)b.num_tokens);
    hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(kThreads), 0, stream, logits, ld, b, k, ws,
                       out, ldo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_resolve_kernel, dim3((unsigned)b.num_tokens), dim3(kRowThreads), 0,
                       stream, logits, ld, b, k, ws, out, ldo);
  } else {
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)b.num_tokens), dim3(kRowThreads), 0,
                       stream, logits, ld, b, k, out, ldo);
  }
  return hipGetLastError();
}

}  // namespace idx

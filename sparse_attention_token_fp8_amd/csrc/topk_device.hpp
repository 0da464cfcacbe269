// Device helpers for the radix top-k (internal): a 256-thread block scan and
// the level-1 threshold pick that runs in the last work-group of a row.
#pragma once

#include "common.hpp"

namespace idx {

constexpr int kThreads = 256;

// Exclusive prefix sum of one value per thread over a 256-thread block.
// `scratch` holds at least 4 words of LDS.  All threads must call it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total,
                                                         uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    const uint32_t s = scratch[i];
    before += (i < wave) ? s : 0u;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// Given the complete level-1 histogram of row t (hist[t][*], updated with
// atomics by other work-groups), find the digit b1 holding the k-th largest
// key: #(digit > b1) < k <= #(digit >= b1).  Writes b1, need = k - #(digit > b1)
// and cand_total = hist[b1] into the row state.  Called by all 256 threads of
// the last work-group after an acquire fence.
__device__ __forceinline__ void pick_threshold(const TopkWorkspace& ws, int t, int k,
                                               uint32_t* scratch) {
  const uint32_t* h = ws.hist + (size_t)t * kBins1;
  constexpr int kPer = kBins1 / kThreads;  // 8 digits per thread, descending
  const int top = kBins1 - 1 - kPer * (int)threadIdx.x;
  uint32_t c[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = load_agent(h + (top - j));
    sum += c[j];
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan(sum, &total, scratch);
  if (before < (uint32_t)k && before + sum >= (uint32_t)k) {
    uint32_t cum = before;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (cum + c[j] >= (uint32_t)k) {
        RowState* st = ws.state + t;
        st->b1 = (uint32_t)(top - j);
        st->need = (uint32_t)k - cum;
        st->cand_total = c[j];
        break;
      }
      cum += c[j];
    }
  }
}

// Flush a work-group's LDS histogram into row t's global histogram, then
// count this work-group as done; the last of `chunks` work-groups picks the
// threshold.  All threads must call it.
__device__ __forceinline__ void finish_hist(const TopkWorkspace& ws, int t, int k, int chunks,
                                            const uint32_t* lhist, uint32_t* scratch) {
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)t * kBins1;
  for (int i = threadIdx.x; i < kBins1; i += kThreads) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(gh + i, v);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&ws.state[t].done_hist, 1u);
    scratch[4] = (prev == (uint32_t)(chunks - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (scratch[4]) {
    __threadfence();
    pick_threshold(ws, t, k, scratch);
  }
}

}  // namespace idx

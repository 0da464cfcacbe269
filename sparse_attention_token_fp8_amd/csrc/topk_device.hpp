// Device building blocks of the top-k select (internal).
//
// Selection rule (IndexCache blog post: the persistent topk_indices_buffer is
// int32 [tokens, index_topk], entries not produced are -1): the k largest
// scores among positions 0..p_t, ties to the lower position, -0 == +0; the row
// lists the selected positions ascending, then -1.
//
// Scores become order-preserving 32-bit keys.  The exact k-th largest key K*
// among a candidate set is found with three LDS histogram passes over digits
// [31:21], [20:10], [9:0].  Candidates are every key >= tau, where tau is the
// j-th largest key of a fixed sample of the row chosen so that almost surely at
// least k keys pass; if fewer do, the whole row is the candidate set, so the
// result never depends on tau.  The row is written through an LDS bitmap:
// keys > K* are set, keys == K* are set in position order until k are taken.
#pragma once

#include "common.hpp"

namespace idx {

constexpr int kThreads = 256;

template <int NT>
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* total, uint32_t* scratch) {
  constexpr int NW = NT / 64;
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
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = scratch[i];
    before += (i < wave) ? s : 0u;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// 256-thread form kept for the small kernels.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total,
                                                         uint32_t* scratch) {
  return block_scan_excl<kThreads>(v, total, scratch);
}

// In an LDS histogram h[0..nb) find the digit d, searching from the top, with
// #(digit > d) < need <= #(digit >= d).  Returns d to every thread and sets
// *above = #(digit > d).  If the histogram holds fewer than `need` entries the
// result is digit 0 with *above = total.
template <int NT>
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, int nb, uint32_t need,
                                               uint32_t* above, uint32_t* scratch) {
  const int per = nb / NT > 0 ? nb / NT : 1;
  const int active = nb / per;            // threads that own digits
  const int top = nb - 1 - per * (int)threadIdx.x;
  uint32_t sum = 0;
  if ((int)threadIdx.x < active)
    for (int j = 0; j < per; ++j) sum += h[top - j];
  if (threadIdx.x == 0) { scratch[NT / 64 + 1] = 0u; scratch[NT / 64 + 2] = 0u; }
  uint32_t total;
  const uint32_t before = block_scan_excl<NT>(sum, &total, scratch);
  if ((int)threadIdx.x < active && before < need && before + sum >= need) {
    uint32_t cum = before;
    for (int j = 0; j < per; ++j) {
      const uint32_t c = h[top - j];
      if (cum + c >= need) {
        scratch[NT / 64 + 1] = (uint32_t)(top - j);
        scratch[NT / 64 + 2] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  uint32_t d = scratch[NT / 64 + 1];
  *above = scratch[NT / 64 + 2];
  if (total < need) { d = 0; *above = total; }
  __syncthreads();
  return d;
}

// Exact `need`-th largest key (need >= 1) of the set visited by `visit(fn)`,
// where fn(key, pos) is called once per element, spread over the block.
// Returns K* and sets *take_eq = how many keys equal to K* belong to the top
// `need` (the rest of the top set is every key > K*).  `hist` holds kBins1
// words of LDS.
template <int NT, typename V>
__device__ __forceinline__ uint32_t radix_kth(V&& visit, uint32_t need, uint32_t* take_eq,
                                              uint32_t* hist, uint32_t* scratch) {
  uint32_t prefix = 0;
  // level 1: digit [31:21]
  for (int i = threadIdx.x; i < kBins1; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key, int) { atomicAdd(&hist[key >> kShift1], 1u); });
  __syncthreads();
  uint32_t above;
  const uint32_t d1 = find_digit<NT>(hist, kBins1, need, &above, scratch);
  need -= above;
  prefix = d1;
  // level 2: digit [20:10] among keys with digit1 == d1
  for (int i = threadIdx.x; i < kBins2; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key, int) {
    if ((key >> kShift1) == prefix) atomicAdd(&hist[(key >> kShift2) & (kBins2 - 1)], 1u);
  });
  __syncthreads();
  const uint32_t d2 = find_digit<NT>(hist, kBins2, need, &above, scratch);
  need -= above;
  prefix = (d1 << (kShift1 - kShift2)) | d2;
  // level 3: digit [9:0] among keys with digits (d1, d2)
  for (int i = threadIdx.x; i < kBins3; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key, int) {
    if ((key >> kShift2) == prefix) atomicAdd(&hist[key & (kBins3 - 1)], 1u);
  });
  __syncthreads();
  const uint32_t d3 = find_digit<NT>(hist, kBins3, need, &above, scratch);
  *take_eq = need - above;
  return (prefix << kShift2) | d3;
}

constexpr int kSeg = 65536;             // positions per emission bitmap segment
constexpr int kSegWords = kSeg / 32;

// Write the selected positions of one row in ascending order: every visited
// key > kstar, plus the first `take_eq` positions (in position order) whose key
// equals kstar; then -1 up to k.  `bits` holds 2*kSegWords words of LDS.
template <int NT, typename V>
__device__ __forceinline__ void emit_row(V&& visit, int n, uint32_t kstar, uint32_t take_eq, int k,
                                         int32_t* __restrict__ out, uint32_t* bits,
                                         uint32_t* scratch) {
  constexpr int kWordsPerThread = kSegWords / NT;
  uint32_t* sel = bits;
  uint32_t* tie = bits + kSegWords;
  uint32_t written = 0, ties_taken = 0;
  for (int g0 = 0; g0 < n; g0 += kSeg) {
    for (int i = threadIdx.x; i < 2 * kSegWords; i += NT) bits[i] = 0;
    __syncthreads();
    visit([&](uint32_t key, int pos) {
      const int s = pos - g0;
      if (s < 0 || s >= kSeg) return;
      if (key > kstar) atomicOr(&sel[s >> 5], 1u << (s & 31));
      else if (key == kstar) atomicOr(&tie[s >> 5], 1u << (s & 31));
    });
    __syncthreads();
    const int w0 = threadIdx.x * kWordsPerThread;
    uint32_t my_ties = 0;
    for (int j = 0; j < kWordsPerThread; ++j) my_ties += __popc(tie[w0 + j]);
    uint32_t seg_ties;
    uint32_t tb = ties_taken + block_scan_excl<NT>(my_ties, &seg_ties, scratch);
    for (int j = 0; j < kWordsPerThread; ++j) {
      uint32_t word = tie[w0 + j];
      while (word) {
        const uint32_t bit = word & (0u - word);
        word ^= bit;
        if (tb < take_eq) sel[w0 + j] |= bit;
        ++tb;
      }
    }
    ties_taken += seg_ties;
    uint32_t my_sel = 0;
    for (int j = 0; j < kWordsPerThread; ++j) my_sel += __popc(sel[w0 + j]);
    uint32_t seg_sel;
    uint32_t o = written + block_scan_excl<NT>(my_sel, &seg_sel, scratch);
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
  for (uint32_t i = written + threadIdx.x; i < (uint32_t)k; i += NT) out[i] = -1;
}

// Sample of a row used to place tau: positions j*S + ((37*j + 11) & (S-1)),
// S a power of two chosen so that at most kMaxSample positions are drawn.
constexpr int kMaxSample = 2048;

__device__ __forceinline__ int sample_stride(int n) {
  int S = 16;
  while ((n + S - 1) / S > kMaxSample) S <<= 1;
  return S;
}

__device__ __forceinline__ int sample_pos(int j, int S) { return j * S + ((37 * j + 11) & (S - 1)); }

// Rank (1-based) of the sample key used as tau: about 2k of the n keys are
// expected at or above it, plus a margin of 16 sample steps.
__device__ __forceinline__ uint32_t sample_rank(int n, int ns, int k) {
  const int64_t j = ((int64_t)2 * k * ns + n - 1) / n + 16;
  return (uint32_t)(j < ns ? j : ns);
}

// tau for one row: 0 (every key passes) when n <= all_below, else the
// sample_rank-th largest sampled key.  Every thread of the block gets it.
template <int NT>
__device__ __forceinline__ uint32_t row_tau(const float* __restrict__ row, int n, int k, int all_below,
                                            uint32_t* hist, uint32_t* scratch) {
  if (n <= all_below) return 0u;
  const int S = sample_stride(n);
  constexpr int kPer = (kMaxSample + NT - 1) / NT;
  uint32_t keys[kPer];
  int ns = 0;
  // number of sample positions inside the row
  {
    const int jmax = (n + S - 1) / S;
    ns = jmax;
    if (jmax > 0 && sample_pos(jmax - 1, S) >= n) ns = jmax - 1;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int j = threadIdx.x + e * NT;
    keys[e] = j < ns ? order_key(row[sample_pos(j, S)]) : 0u;
  }
  const uint32_t j = sample_rank(n, ns, k);
  uint32_t take;
  return radix_kth<NT>([&](auto&& fn) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int jj = threadIdx.x + e * NT;
      if (jj < ns) fn(keys[e], jj);
    }
  }, j, &take, hist, scratch);
}

}  // namespace idx

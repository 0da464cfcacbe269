// Device building blocks of the top-k select (internal).
//
// Selection rule (IndexCache blog post: the persistent topk_indices_buffer is
// int32 [tokens, index_topk], entries not produced are -1): the k largest
// scores among positions 0..p_t, ties to the lower position, -0 == +0; the row
// lists the selected positions ascending, then -1.
//
// Scores become order-preserving 32-bit keys.  Candidates are every key >=
// tau, where tau comes from a fixed sample of the row and is placed so that
// almost surely at least k keys pass; if fewer do, the whole row is the
// candidate set, so the result never depends on tau.  The exact k-th largest
// key K* among the candidates comes from LDS histograms whose digits are taken
// relative to the smallest candidate (a narrow score band then spreads over
// the bins); once the band holding K* has at most 64 keys, one wave ranks them
// directly.  Candidates are kept in ascending position order, so the row is
// written with one block-wide scan: a candidate's output slot is
// #(earlier keys > K*) + min(#(earlier keys == K*), take_eq).
#pragma once

#include "common.hpp"

namespace idx {

constexpr int kThreads = 256;

// LEAD: synchronise before writing `scratch`, for callers whose threads may
// still be reading it from an earlier scan.
template <int NT, bool LEAD = true>
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* total, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (LEAD) __syncthreads();
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

// 64-bit form: `scratch` holds at least 2*NT/64 words.
template <int NT>
__device__ __forceinline__ uint64_t block_scan_excl64(uint64_t v, uint64_t* total, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)incl, off, 64);
    const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(incl >> 32), off, 64);
    if (lane >= off) incl += ((uint64_t)hi << 32) | lo;
  }
  __syncthreads();
  if (lane == 63) { scratch[2 * wave] = (uint32_t)incl; scratch[2 * wave + 1] = (uint32_t)(incl >> 32); }
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint64_t s = ((uint64_t)scratch[2 * i + 1] << 32) | scratch[2 * i];
    before += (i < wave) ? s : 0ull;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// Words of LDS scratch the helpers below need for an NT-thread block.
template <int NT>
constexpr int scratch_words() { return 2 * (NT / 64) + 8; }

// In an LDS histogram h[0..nb) find the digit d, searching from the top, with
// #(digit > d) < need <= #(digit >= d).  Returns d to every thread and sets
// *above = #(digit > d) and *count = h[d].  If the histogram holds fewer than
// `need` entries the result is digit 0 with *above = total.
template <int NT>
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, int nb, uint32_t need,
                                               uint32_t* above, uint32_t* scratch,
                                               uint32_t* count = nullptr) {
  const int per = nb / NT > 0 ? nb / NT : 1;
  const int active = nb / per;
  const int top = nb - 1 - per * (int)threadIdx.x;
  uint32_t sum = 0;
  if ((int)threadIdx.x < active)
    for (int j = 0; j < per; ++j) sum += h[top - j];
  uint32_t* res = scratch + NT / 64;
  if (threadIdx.x == 0) { res[1] = 0u; res[2] = 0u; res[3] = 0u; }
  uint32_t total;
  // Every caller has synchronised after filling `h` (so after any earlier
  // reads of `scratch`): the scan needs no leading barrier.
  const uint32_t before = block_scan_excl<NT, false>(sum, &total, scratch);
  if ((int)threadIdx.x < active && before < need && before + sum >= need) {
    uint32_t cum = before;
    for (int j = 0; j < per; ++j) {
      const uint32_t c = h[top - j];
      if (cum + c >= need) {
        res[1] = (uint32_t)(top - j);
        res[2] = cum;
        res[3] = c;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  uint32_t d = res[1];
  *above = res[2];
  if (count) *count = res[3];
  if (total < need) { d = 0; *above = total; }
  __syncthreads();
  return d;
}

// The `need`-th largest key (need >= 1) of the set visited by `visit(fn)`,
// where fn(key) is called once per element, spread over the block.  With
// LEVELS == 3 the result is exact and *take_eq = how many keys equal to it
// belong to the top `need`; with LEVELS == 2 the result is the key rounded
// down to a multiple of 2^10 (enough for placing a threshold).
// `hist` holds kBins1 words of LDS.
template <int NT, int LEVELS, typename V>
__device__ __forceinline__ uint32_t radix_kth(V&& visit, uint32_t need, uint32_t* take_eq,
                                              uint32_t* hist, uint32_t* scratch) {
  for (int i = threadIdx.x; i < kBins1; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key) { atomicAdd(&hist[key >> kShift1], 1u); });
  __syncthreads();
  uint32_t above;
  const uint32_t d1 = find_digit<NT>(hist, kBins1, need, &above, scratch);
  need -= above;
  for (int i = threadIdx.x; i < kBins2; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key) {
    if ((key >> kShift1) == d1) atomicAdd(&hist[(key >> kShift2) & (kBins2 - 1)], 1u);
  });
  __syncthreads();
  const uint32_t d2 = find_digit<NT>(hist, kBins2, need, &above, scratch);
  need -= above;
  const uint32_t prefix = (d1 << (kShift1 - kShift2)) | d2;
  if (LEVELS == 2) {
    *take_eq = 0;
    return prefix << kShift2;
  }
  for (int i = threadIdx.x; i < kBins3; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key) {
    if ((key >> kShift2) == prefix) atomicAdd(&hist[key & (kBins3 - 1)], 1u);
  });
  __syncthreads();
  const uint32_t d3 = find_digit<NT>(hist, kBins3, need, &above, scratch);
  *take_eq = need - above;
  return (prefix << kShift2) | d3;
}

// Exact `need`-th largest key (1 <= need <= C) of ckey[0..C) in LDS, with
// *take_eq = how many keys equal to it belong to the top `need`.  Digits of
// up to 11 bits are taken over [kmin, kmax] of the candidates; when the bin
// holding the answer has at most 64 keys they are ranked by one wave.
// `hist` holds kBins1 words, `bucket` 64 words.  select_kth_range takes the
// range from the caller (every key must lie in [kmin, kmax]).
template <int NT>
__device__ __forceinline__ uint32_t select_kth_range(const uint32_t* ckey, uint32_t C, uint32_t need,
                                                     uint32_t kmin, uint32_t kmax,
                                                     uint32_t* take_eq, uint32_t* hist,
                                                     uint32_t* bucket, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  uint32_t* sx = scratch + 2 * NW;              // bucket fill, K*, take
  uint32_t base = kmin;
  int width = kmax == kmin ? 0 : 32 - __clz(kmax - kmin);   // keys in play: [base, base + 2^width)
  while (width > 0) {
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = 1 << (width - shift);
    for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0;
    if (threadIdx.x == 0) sx[0] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < C; i += NT) {
      const uint32_t x = ckey[i];
      if (x >= base && ((uint64_t)(x - base) >> width) == 0) atomicAdd(&hist[(x - base) >> shift], 1u);
    }
    __syncthreads();
    uint32_t above, in_bin;
    const uint32_t d = find_digit<NT>(hist, nb, need, &above, scratch, &in_bin);
    need -= above;
    base += d << shift;
    width = shift;
    if (width > 0 && in_bin <= 64) {            // rank the bin's keys in one wave
      for (uint32_t i = threadIdx.x; i < C; i += NT) {
        const uint32_t x = ckey[i];
        if (x >= base && ((uint64_t)(x - base) >> width) == 0) {
          const uint32_t j = atomicAdd(&sx[0], 1u);
          if (j < 64u) bucket[j] = x;
        }
      }
      __syncthreads();
      if ((uint32_t)threadIdx.x < in_bin) {
        const uint32_t x = bucket[threadIdx.x];
        uint32_t gt = 0, ge = 0;
        for (uint32_t j = 0; j < in_bin; ++j) {
          const uint32_t y = bucket[j];
          gt += y > x;
          ge += y >= x;
        }
        if (gt < need && need <= ge) { sx[1] = x; sx[2] = need - gt; }
      }
      __syncthreads();
      base = sx[1];
      need = sx[2];
      width = 0;
      __syncthreads();
    }
  }
  *take_eq = need;
  return base;
}

// The same, with the range taken from the keys first.
template <int NT>
__device__ __forceinline__ uint32_t select_kth(const uint32_t* ckey, uint32_t C, uint32_t need,
                                               uint32_t* take_eq, uint32_t* hist, uint32_t* bucket,
                                               uint32_t* scratch) {
  constexpr int NW = NT / 64;
  uint32_t* sx = scratch + 2 * NW + 4;          // kmin, kmax
  const int lane = threadIdx.x & 63;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (uint32_t i = threadIdx.x; i < C; i += NT) {
    const uint32_t x = ckey[i];
    lo = min(lo, x);
    hi = max(hi, x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
  }
  if (threadIdx.x == 0) { sx[0] = 0xffffffffu; sx[1] = 0u; }
  __syncthreads();
  if (lane == 0) { atomicMin(&sx[0], lo); atomicMax(&sx[1], hi); }
  __syncthreads();
  return select_kth_range<NT>(ckey, C, need, sx[0], sx[1], take_eq, hist, bucket, scratch);
}

// Write one row: `get(i)` returns (key, position) of the i-th of `count`
// elements, in ascending position order.  Keys > kstar are taken, and the
// first take_eq keys == kstar; the rest of the k slots get -1.
template <int NT, typename G>
__device__ __forceinline__ void emit_ordered(G&& get, uint32_t count, uint32_t kstar, uint32_t take_eq,
                                             int k, int32_t* __restrict__ out, uint32_t* scratch) {
  const uint32_t per = (count + NT - 1) / NT;
  const uint32_t i0 = min(count, per * threadIdx.x), i1 = min(count, i0 + per);
  uint32_t gt = 0, eq = 0;
  for (uint32_t i = i0; i < i1; ++i) {
    const uint32_t key = get(i).x;
    gt += key > kstar;
    eq += key == kstar;
  }
  uint32_t gb, eb, gall, eall;
  if (count < 65536u) {                         // both counts fit 16 bits: one 32-bit scan
    uint32_t total;
    const uint32_t pre = block_scan_excl<NT>((eq << 16) | gt, &total, scratch);
    gb = pre & 0xffffu; eb = pre >> 16;
    gall = total & 0xffffu; eall = total >> 16;
  } else {
    uint64_t total;
    const uint64_t pre = block_scan_excl64<NT>(((uint64_t)eq << 32) | gt, &total, scratch);
    gb = (uint32_t)pre; eb = (uint32_t)(pre >> 32);
    gall = (uint32_t)total; eall = (uint32_t)(total >> 32);
  }
  for (uint32_t i = i0; i < i1; ++i) {
    const uint2 kp = get(i);
    if (kp.x > kstar) {
      const uint32_t o = gb + min(eb, take_eq);
      if (o < (uint32_t)k) out[o] = (int32_t)kp.y;
      ++gb;
    } else if (kp.x == kstar) {
      if (eb < take_eq && gb + eb < (uint32_t)k) out[gb + eb] = (int32_t)kp.y;
      ++eb;
    }
  }
  const uint32_t written = min((uint32_t)k, gall + min(eall, take_eq));
  for (uint32_t i = written + threadIdx.x; i < (uint32_t)k; i += NT) out[i] = -1;
  __syncthreads();
}

// Rank (1-based) of the sample key used as tau: about 1.5k of the n keys are
// expected at or above it, plus a margin of 16 sample steps (the count stays
// several standard deviations above k for samples of a few hundred keys).
__device__ __forceinline__ uint32_t sample_rank(int n, int ns, int k) {
  const int64_t j = ((int64_t)3 * k * ns + 2 * (int64_t)n - 1) / (2 * (int64_t)n) + 16;
  return (uint32_t)(j < ns ? j : ns);
}

template <int NT>
constexpr int sample_per() { return (kMaxSample + NT - 1) / NT; }

// Issue the loads of the row's sample into v[sample_per<NT>()]; returns the
// sample size.
template <int NT>
__device__ __forceinline__ int sample_load(const float* __restrict__ row, int n, float* v) {
  const int S = sample_stride(n);
  int ns = (n + S - 1) / S;
  if (ns > 0 && sample_pos(ns - 1, S) >= n) --ns;
#pragma unroll
  for (int e = 0; e < sample_per<NT>(); ++e) {
    const int j = threadIdx.x + e * NT;
    v[e] = j < ns ? row[sample_pos(j, S)] : 0.f;
  }
  return ns;
}

// The same sample read from a compact copy (entry j = the score at
// sample_pos(j, S)) that the scoring kernel wrote.
template <int NT>
__device__ __forceinline__ int sample_load_compact(const float* __restrict__ samp, int n, float* v) {
  const int S = sample_stride(n);
  int ns = (n + S - 1) / S;
  if (ns > 0 && sample_pos(ns - 1, S) >= n) --ns;
#pragma unroll
  for (int e = 0; e < sample_per<NT>(); ++e) {
    const int j = threadIdx.x + e * NT;
    v[e] = j < ns ? samp[j] : 0.f;
  }
  return ns;
}

// tau from the loaded sample: the sample_rank-th largest sampled key rounded
// down to a multiple of 2^10.  Every thread of the block gets it.
template <int NT>
__device__ __forceinline__ uint32_t sample_tau(const float* v, int ns, int n, int k, uint32_t* hist,
                                               uint32_t* scratch) {
  uint32_t take;
  return radix_kth<NT, 2>([&](auto&& fn) {
#pragma unroll
    for (int e = 0; e < sample_per<NT>(); ++e)
      if ((int)threadIdx.x + e * NT < ns) fn(order_key(v[e]));
  }, sample_rank(n, ns, k), &take, hist, scratch);
}

// Ordered compaction of one batch: element (e, thread) sits at position
// base + e*NT + threadIdx.x; those with pass[e] are appended to (ckey, cpos)
// after `start` entries, in ascending position order (entries past `cap` are
// counted, not stored).  `table` holds E*NT/64 <= 64 words of LDS.  There is
// one barrier: every wave scans the per-(e, wave) counts itself.  So two
// consecutive calls must not share a table (callers alternate two), and a
// caller synchronises before it reads what was compacted into LDS.  Returns
// the batch's number of passing elements.
template <int NT, int E, typename Pos>
__device__ __forceinline__ uint32_t compact_ordered(const uint32_t* key, const bool* pass, int base,
                                                    uint32_t start, uint32_t* ckey, Pos* cpos,
                                                    uint32_t cap, uint32_t* table) {
  constexpr int NW = NT / 64;
  static_assert(E * NW <= 64, "one count per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  uint64_t m[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    m[e] = __ballot(pass[e]);
    if (lane == 0) table[e * NW + wave] = (uint32_t)__popcll(m[e]);
  }
  __syncthreads();
  // exclusive prefix over the E*NW counts in (e, wave) order, lane i holding count i
  const uint32_t c = lane < E * NW ? table[lane] : 0u;
  uint32_t incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
    if (lane >= off) incl += y;
  }
  const uint32_t excl = incl - c;
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)excl, e * NW + wave);
    if (pass[e]) {
      const uint32_t slot = start + at + (uint32_t)__popcll(m[e] & below);
      if (slot < cap) { ckey[slot] = key[e]; cpos[slot] = (Pos)(base + e * NT + (int)threadIdx.x); }
    }
  }
  return total;
}

}  // namespace idx

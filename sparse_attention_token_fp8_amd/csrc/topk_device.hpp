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
  const uint32_t incl = wave_sum_incl(v);
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

// In an LDS histogram h[0..nb), nb a power of two <= 2048, the digit d,
// searched from the top, with #(digit > d) < need <= #(digit >= d): found by
// one wave on its own (every wave of a block gets the same answer, with no
// barrier).  Lane l sums the bins [nb - per(l+1), nb - per*l), per =
// max(nb/64, 1) (lanes in descending key order; reads rotated by lane so that
// few lanes of a pass hit one bank), one scan finds the lane whose bins reach
// `need`, a second scan that lane's bins.  Sets *above = #(digit > d), *count = h[d] and
// *total; with fewer than `need` entries the result is digit 0, *above = total.
__device__ __forceinline__ uint32_t wave_digit(const uint32_t* h, int nb, uint32_t need,
                                               uint32_t* above, uint32_t* count, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int per = nb >= 64 ? nb / 64 : 1;
  const int active = nb >= 64 ? 64 : nb;
  uint32_t sum = 0u;
  if (lane < active) {
    // all kBins1/64 reads unconditional (indices wrap inside the lane's bins),
    // so they are issued together whatever `per` is
    const uint32_t* hb = h + nb - per * (lane + 1);
    uint32_t v[kBins1 / 64];
#pragma unroll
    for (int i = 0; i < kBins1 / 64; ++i) v[i] = hb[(i + lane) & (per - 1)];
#pragma unroll
    for (int i = 0; i < kBins1 / 64; ++i) sum += i < per ? v[i] : 0u;
  }
  const uint32_t incl = wave_sum_incl(sum);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  *total = tot;
  if (tot < need) {
    *above = tot;
    *count = 0u;
    return 0u;
  }
  const int L = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;
  const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
  const uint32_t* hl = h + nb - per * (L + 1);
  const uint32_t c = lane < per ? hl[per - 1 - lane] : 0u;   // lane j: the lane's j-th highest bin
  const uint32_t inc2 = wave_sum_incl(c);
  const int j = __ffsll((unsigned long long)__ballot(lane < per && before + inc2 >= need)) - 1;
  *above = before + (uint32_t)__builtin_amdgcn_readlane((int)(inc2 - c), j);
  *count = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
  return (uint32_t)(nb - per * (L + 1) + (per - 1 - j));
}

// wave_digit for a block of NT threads, every thread getting the answer: up
// to four waves each search on their own; larger blocks let wave 0 search and
// pass the result through `scratch` (four words) and one barrier.  Callers
// synchronise before they reuse `h`.
template <int NT>
__device__ __forceinline__ uint32_t block_digit(const uint32_t* h, int nb, uint32_t need,
                                                uint32_t* above, uint32_t* count, uint32_t* total,
                                                uint32_t* scratch) {
  if (NT <= 256) return wave_digit(h, nb, need, above, count, total);
  if (threadIdx.x < 64) {
    uint32_t a, c, t;
    const uint32_t d = wave_digit(h, nb, need, &a, &c, &t);
    if (threadIdx.x == 0) { scratch[0] = d; scratch[1] = a; scratch[2] = c; scratch[3] = t; }
  }
  __syncthreads();
  *above = scratch[1];
  *count = scratch[2];
  *total = scratch[3];
  return scratch[0];
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
  uint32_t above, cnt, total;
  for (int i = threadIdx.x; i < kBins1; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key) { atomicAdd(&hist[key >> kShift1], 1u); });
  __syncthreads();
  const uint32_t d1 = block_digit<NT>(hist, kBins1, need, &above, &cnt, &total, scratch + NT / 64);
  need -= above;
  __syncthreads();                              // every wave has read the histogram
  for (int i = threadIdx.x; i < kBins2; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key) {
    if ((key >> kShift1) == d1) atomicAdd(&hist[(key >> kShift2) & (kBins2 - 1)], 1u);
  });
  __syncthreads();
  const uint32_t d2 = block_digit<NT>(hist, kBins2, need, &above, &cnt, &total, scratch + NT / 64);
  need -= above;
  const uint32_t prefix = (d1 << (kShift1 - kShift2)) | d2;
  if (LEVELS == 2) {
    *take_eq = 0;
    __syncthreads();                            // the histogram is free for the caller
    return prefix << kShift2;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins3; i += NT) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t key) {
    if ((key >> kShift2) == prefix) atomicAdd(&hist[key & (kBins3 - 1)], 1u);
  });
  __syncthreads();
  const uint32_t d3 = block_digit<NT>(hist, kBins3, need, &above, &cnt, &total, scratch + NT / 64);
  *take_eq = need - above;
  __syncthreads();                              // the histogram is free for the caller
  return (prefix << kShift2) | d3;
}

// fn(ckey[i]) for i = threadIdx.x, threadIdx.x + NT, ... < C, the reads of
// four iterations issued together (a loop that uses each LDS read at once
// would wait for every read in turn).
template <int NT, typename F>
__device__ __forceinline__ void for_keys(const uint32_t* ckey, uint32_t C, F&& fn) {
  constexpr int U = 4;
  for (uint32_t i = threadIdx.x; i < C; i += U * NT) {
    uint32_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = ckey[min(i + u * NT, C - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + u * NT < C) fn(x[u]);
  }
}

// Exact `need`-th largest key (1 <= need <= C) of ckey[0..C) in LDS, with
// *take_eq = how many keys equal to it belong to the top `need`.  Digits of
// up to 11 bits are taken over [kmin, kmax] of the candidates; when the bin
// holding the answer has at most 64 keys they are ranked by one wave.
// `hist` holds kBins1 words, `bucket` 64 words.  select_kth_range takes the
// range from the caller: keys outside [kmin, kmax] are ignored.
// With in_range, *in_range receives the number of keys in [kmin, kmax]; when
// it is below `need` nothing more is done and the result is meaningless.
// ZERO_FIRST = false: the caller has cleared hist[0..kBins1) and synchronised.
template <int NT, bool ZERO_FIRST = true>
__device__ __forceinline__ uint32_t select_kth_range(const uint32_t* ckey, uint32_t C, uint32_t need,
                                                     uint32_t kmin, uint32_t kmax,
                                                     uint32_t* take_eq, uint32_t* hist,
                                                     uint32_t* bucket, uint32_t* scratch,
                                                     uint32_t* in_range = nullptr) {
  constexpr int NW = NT / 64;
  uint32_t* sx = scratch + 2 * NW;              // bucket fill, K*, take, count
  uint32_t base = kmin;
  int width = kmax == kmin ? 0 : 32 - __clz(kmax - kmin);   // keys in play: [base, base + 2^width)
  if (in_range != nullptr && width == 0) {      // every key in play equals kmin: count them
    if (threadIdx.x == 0) sx[3] = 0u;
    __syncthreads();
    uint32_t c = 0;
    for_keys<NT>(ckey, C, [&](uint32_t x) { c += x == kmin; });
    c = wave_sum(c);
    if ((threadIdx.x & 63) == 0) atomicAdd(&sx[3], c);
    __syncthreads();
    *in_range = sx[3];
    __syncthreads();
  }
  bool first = true;
  while (width > 0) {
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = 1 << (width - shift);
    if (!first) __syncthreads();                // every wave is done with the last pass's bins
    if (ZERO_FIRST || !first)
      for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0;
    if (threadIdx.x == 0) sx[0] = 0u;
    __syncthreads();
    for_keys<NT>(ckey, C, [&](uint32_t x) {
      if (x >= base && ((uint64_t)(x - base) >> width) == 0) atomicAdd(&hist[(x - base) >> shift], 1u);
    });
    __syncthreads();
    uint32_t above, in_bin, total;
    const uint32_t d = block_digit<NT>(hist, nb, need, &above, &in_bin, &total, scratch + NW);
    if (first && in_range != nullptr) {
      *in_range = total;
      if (total < need) {                       // uniform: every thread has the same total
        *take_eq = 0;
        return base;
      }
    }
    first = false;
    need -= above;
    base += d << shift;
    width = shift;
    if (width > 0 && in_bin <= 64) {            // rank the bin's keys in one wave
      for_keys<NT>(ckey, C, [&](uint32_t x) {
        if (x >= base && ((uint64_t)(x - base) >> width) == 0) {
          const uint32_t j = atomicAdd(&sx[0], 1u);
          if (j < 64u) bucket[j] = x;
        }
      });
      __syncthreads();
      if (threadIdx.x < 64) {                   // wave 0: lane j holds bucket[j], ranks by readlane
        const int lane = threadIdx.x;
        const uint32_t x = (uint32_t)lane < in_bin ? bucket[lane] : 0u;
        uint32_t gt = 0, ge = 0;
        for (int j = 0; j < (int)in_bin; ++j) {
          const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, j);
          gt += y > x;
          ge += y >= x;
        }
        if ((uint32_t)lane < in_bin && gt < need && need <= ge) { sx[1] = x; sx[2] = need - gt; }
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
  lo = wave_min(lo);
  hi = wave_max(hi);
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
  constexpr int U = 4;                          // reads of four elements issued together
  uint32_t gt = 0, eq = 0;
  for (uint32_t i = i0; i < i1; i += U) {
    uint32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) key[u] = get(min(i + u, i1 - 1)).x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      gt += i + u < i1 && key[u] > kstar;
      eq += i + u < i1 && key[u] == kstar;
    }
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
  for (uint32_t i = i0; i < i1; i += U) {
    uint2 kp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kp[u] = get(min(i + u, i1 - 1));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u >= i1) break;
      if (kp[u].x > kstar) {
        const uint32_t o = gb + min(eb, take_eq);
        if (o < (uint32_t)k) out[o] = (int32_t)kp[u].y;
        ++gb;
      } else if (kp[u].x == kstar) {
        if (eb < take_eq && gb + eb < (uint32_t)k) out[gb + eb] = (int32_t)kp[u].y;
        ++eb;
      }
    }
  }
  const uint32_t written = min((uint32_t)k, gall + min(eall, take_eq));
  for (uint32_t i = written + threadIdx.x; i < (uint32_t)k; i += NT) out[i] = -1;
  __syncthreads();
}

// The row's k entries from runs of candidates held in registers: wave w
// holds candidates a0 + 64 e + lane < a1 of the row's candidate order
// (ascending positions), the runs of the waves following each other in wave
// order.  Keys > kstar are taken, and the first take_eq keys == kstar; slots
// past those get -1.  Each wave counts its run with ballots, one barrier
// exchanges the counts (`counts`: 2 * NT / 64 words of LDS no other wave is
// reading), and each taken key's position goes to
// #(earlier keys > kstar) + min(#(earlier keys == kstar), take_eq).
template <int NT, int E>
__device__ __forceinline__ void emit_runs(const uint32_t (&key)[E], const int32_t (&pos)[E], uint32_t a0,
                                          uint32_t a1, uint32_t kstar, uint32_t take_eq, int k,
                                          int32_t* __restrict__ out, uint32_t* counts) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int ne = (int)((a1 - a0 + 63u) / 64u);  // uniform
  auto valid = [&](int e) { return a0 + 64u * e + lane < a1; };
  uint32_t ng = 0u, nq = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e < ne) {                               // uniform
      ng += (uint32_t)__popcll(__ballot(valid(e) && key[e] > kstar));
      nq += (uint32_t)__popcll(__ballot(valid(e) && key[e] == kstar));
    }
  }
  if (lane == 0) { counts[2 * wave] = ng; counts[2 * wave + 1] = nq; }
  __syncthreads();
  uint32_t gb = 0u, eb = 0u, gall = 0u, eall = 0u;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint32_t g = counts[2 * v], q = counts[2 * v + 1];
    gb += v < wave ? g : 0u;
    eb += v < wave ? q : 0u;
    gall += g;
    eall += q;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= ne) continue;                      // uniform
    const bool g = valid(e) && key[e] > kstar, q = valid(e) && key[e] == kstar;
    const uint64_t bg = __ballot(g), be = __ballot(q);
    const uint32_t pg = __builtin_amdgcn_mbcnt_hi((uint32_t)(bg >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bg, 0u));
    const uint32_t pe = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
    uint32_t o = 0xffffffffu;
    if (g) o = gb + pg + min(eb + pe, take_eq);
    else if (q && eb + pe < take_eq) o = gb + pg + eb + pe;
    if (o < (uint32_t)k) out[o] = pos[e];
    gb += (uint32_t)__popcll(bg);
    eb += (uint32_t)__popcll(be);
  }
  const uint32_t written = min((uint32_t)k, gall + min(eall, take_eq));
  for (uint32_t i = written + threadIdx.x; i < (uint32_t)k; i += NT) out[i] = -1;
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
// base + e*NT + threadIdx.x; those with pass[e] are handed to put(slot, key,
// position) with slot = start + their rank in ascending position order (put
// drops slots past its capacity; they are still counted).  `table` holds
// E*NT/64 <= 64 words of LDS.  There is one barrier: every wave scans the
// per-(e, wave) counts itself.  So two consecutive calls must not share a
// table (callers alternate two), and a caller synchronises before it reads
// what was compacted into LDS.  Returns the batch's number of passing
// elements.
template <int NT, int E, typename Put>
__device__ __forceinline__ uint32_t compact_ordered_to(const uint32_t* key, const bool* pass, int base,
                                                       uint32_t start, uint32_t* table, Put&& put) {
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
  const uint32_t incl = wave_sum_incl(c);
  const uint32_t excl = incl - c;
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)excl, e * NW + wave);
    if (pass[e])
      put(start + at + (uint32_t)__popcll(m[e] & below), key[e], base + e * NT + (int)threadIdx.x);
  }
  return total;
}

// The same into separate key and position arrays of `cap` entries.
template <int NT, int E, typename Pos>
__device__ __forceinline__ uint32_t compact_ordered(const uint32_t* key, const bool* pass, int base,
                                                    uint32_t start, uint32_t* ckey, Pos* cpos,
                                                    uint32_t cap, uint32_t* table) {
  return compact_ordered_to<NT, E>(key, pass, base, start, table,
                                   [&](uint32_t slot, uint32_t k, int pos) {
                                     if (slot < cap) { ckey[slot] = k; cpos[slot] = (Pos)pos; }
                                   });
}

}  // namespace idx

// Top-k select over the causal scores of each query token (see
// topk_device.hpp for the rule and the method).  Two launch shapes:
//
//   many rows     one 512-thread work-group per row: tau from the row's
//                 sample, candidates (key >= tau) compacted into LDS in
//                 position order, exact select, ordered write-out.  No global
//                 scratch and no atomics outside LDS.  Rows whose sample the
//                 scoring kernel copied out are streamed one contiguous range
//                 per wave (each wave compacting into its own part of the
//                 list); rows whose sample is gathered here are streamed by
//                 the whole work-group, batch by batch.
//   few long rows filter: work-groups of 2048 or 4096 positions compact their
//                 candidates, in order, into a private slot of the workspace
//                 (no atomics, nothing to clear); resolve: one work-group per
//                 row gathers the slots in order and finishes as above.
//
// Neither shape uses device-scope atomics or fences: work-groups meet only at
// kernel boundaries.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "topk_device.hpp"

namespace idx {
namespace {

constexpr int kRowThreads = 512;
constexpr int kCandCap = 6144;       // LDS candidate capacity of the resolve
constexpr int kBatch = 8;            // positions per thread per batch in the row kernel
// Positions per filter work-group.  With the scoring kernel's compact sample
// copy each work-group's tau costs one contiguous 8 KiB read, so smaller chunks
// (more work-groups per CU to hide the latency chains) pay; without it every
// work-group gathers the sample from the row, and larger chunks do better.
constexpr int kChunkSampled = 2048;
constexpr int kChunkPlain = 4096;
constexpr int kMaxLongRow = 1 << 22;                 // rows up to 4M positions
static_assert(kMaxLongRow / kChunkSampled <= kMaxSlots, "one slot per chunk");

// byte_rsrc from wave-uniform values, so that the descriptor sits in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return byte_rsrc(reinterpret_cast<const void*>((uintptr_t)(((uint64_t)hi << 32) | lo)),
                   __builtin_amdgcn_readfirstlane(bytes));
}

template <int NT>
__device__ __forceinline__ void write_all(int32_t* out, int n, int k) {
  for (int j = threadIdx.x; j < k; j += NT) out[j] = j < n ? j : -1;
}

// The ordered write-out of one row from C candidates in LDS (ascending
// positions), by waves: wave w takes a contiguous run of them into registers
// and emit_runs writes the row (`counts`: 2 * NT / 64 words of LDS used by
// nothing else).
template <int NT, typename Pos>
__device__ __forceinline__ void emit_by_waves(const uint32_t* ckey, const Pos* cpos, uint32_t C,
                                              uint32_t kstar, uint32_t take_eq, int k,
                                              int32_t* __restrict__ out, uint32_t* counts) {
  constexpr int NW = NT / 64, E = kRowCap / NT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const uint32_t run = (C + 64 * NW - 1) / (64 * NW) * 64;
  const uint32_t a0 = min(C, (uint32_t)wave * run), a1 = min(C, a0 + run);
  uint32_t key[E];
  int32_t pos[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {                 // every read issued together (in bounds)
    const uint32_t j = min(a0 + 64u * e + lane, C - 1u);
    key[e] = ckey[j];
    pos[e] = (int32_t)cpos[j];
  }
  emit_runs<NT, E>(key, pos, a0, a1, kstar, take_eq, k, out, counts);
}

// Exact select over the `C` candidates in LDS (k <= C <= cap, ascending
// positions), else over the whole row, then the ordered write-out.
template <int NT, typename Pos>
__device__ __forceinline__ void finish_row(const float* __restrict__ row, int n, int k, uint32_t C,
                                           uint32_t cap, const uint32_t* ckey, const Pos* cpos,
                                           int32_t* __restrict__ out, uint32_t* hist,
                                           uint32_t* bucket, uint32_t* scratch) {
  uint32_t take;
  if (C >= (uint32_t)k && C <= cap) {
    const uint32_t kstar = select_kth<NT>(ckey, C, (uint32_t)k, &take, hist, bucket, scratch);
    emit_ordered<NT>([&](uint32_t i) { return make_uint2(ckey[i], (uint32_t)cpos[i]); }, C, kstar,
                     take, k, out, scratch);
  } else {
    const uint32_t kstar = radix_kth<NT, 3>([&](auto&& fn) {
      for (int s = threadIdx.x; s < n; s += NT) fn(order_key(row[s]));
    }, (uint32_t)k, &take, hist, scratch);
    emit_ordered<NT>([&](uint32_t i) { return make_uint2(order_key(row[i]), i); }, (uint32_t)n,
                     kstar, take, k, out, scratch);
  }
}

// tau from the loaded sample (as sample_tau: at or below the sample_rank-th
// largest sampled key) with one histogram: its kBins1 bins of 2^kNearShift
// keys each reach from the largest sampled key M down over four octaves, so
// the bin of the rank-th key gives a threshold within 1/512 of an octave of
// it.  Samples whose rank-th key lies further below M take sample_tau.
constexpr int kNearShift = 14;

template <int NT>
__device__ __forceinline__ uint32_t sample_tau_near_max(const float* v, int ns, int n, int k,
                                                        uint32_t* hist, uint32_t* scratch) {
  constexpr int NW = NT / 64, E = sample_per<NT>();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  uint32_t key[E];
  uint32_t mx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[e] = (int)threadIdx.x + e * NT < ns ? order_key(v[e]) : 0u;
    mx = max(mx, key[e]);
  }
  mx = wave_max(mx);
  for (int i = threadIdx.x; i < kBins1; i += NT) hist[i] = 0u;
  if ((threadIdx.x & 63) == 0) scratch[wave] = mx;
  __syncthreads();
  uint32_t M = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = max(M, scratch[w]);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t d = (M - key[e]) >> kNearShift;   // key <= M: bins ascend towards M
    if ((int)threadIdx.x + e * NT < ns && d < (uint32_t)kBins1) atomicAdd(&hist[kBins1 - 1 - d], 1u);
  }
  __syncthreads();
  const uint32_t rank = sample_rank(n, ns, k);
  uint32_t above, cnt, total;
  const uint32_t dig = block_digit<NT>(hist, kBins1, rank, &above, &cnt, &total, scratch + NW);
  __syncthreads();                              // every wave is done with hist and scratch
  if (total < rank) return sample_tau<NT>(v, ns, n, k, hist, scratch);   // uniform
  // the bin's keys: M - (d + 1) 2^s < key <= M - d 2^s, d = kBins1 - 1 - dig
  const uint64_t below = (uint64_t)(kBins1 - dig) << kNearShift;
  return (uint64_t)M + 1u > below ? (uint32_t)((uint64_t)M + 1u - below) : 0u;
}

// One work-group per row.  Candidate positions are stored as Pos (16 bits
// when every row fits in 65536 positions), which with 512 threads lets four
// rows share a CU.
// With `samp` (the scoring kernel's compact sample copy) the sample is one
// contiguous read; without it the sampled positions are gathered from the row,
// which touches every line of it once more before the pass over the row.
template <typename Pos, bool RANGES>
__global__ __launch_bounds__(kRowThreads) void topk_rows_kernel(const float* __restrict__ logits,
                                                                int64_t ld, BatchArgs b, int k,
                                                                int32_t* __restrict__ topk,
                                                                int64_t ldo,
                                                                const float* __restrict__ samp) {
  const int t = blockIdx.x;
  float sv[sample_per<kRowThreads>()];
  if constexpr (RANGES) {
    // the compact copy is read whole before the row's length is known, so the
    // two round trips overlap; entries past the row's sample are never used
#pragma unroll
    for (int e = 0; e < sample_per<kRowThreads>(); ++e)
      sv[e] = samp[(size_t)t * kMaxSample + threadIdx.x + e * kRowThreads];
  }
  const int n = token_pos_wave(b, t).n;
  int32_t* out = topk + (size_t)t * ldo;
  if (n <= k) {
    write_all<kRowThreads>(out, n, k);
    return;
  }
  __shared__ uint32_t ckey[kRowCap];
  __shared__ Pos cpos[kRowCap];
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t table[2][kBatch * kRowThreads / 64];   // alternate batches alternate tables
  __shared__ uint32_t bucket[64];
  __shared__ uint32_t scratch[scratch_words<kRowThreads>()];
  const float* row = logits + (size_t)t * ld;
  constexpr int kStep = kRowThreads * kBatch;
  const bool sampled = n > kRowCap;             // else every position is a candidate
  int ns = 0;
  if (sampled) {
    if constexpr (RANGES) {                     // the sample's size (its values are loaded)
      const int S = sample_stride(n);
      ns = (n + S - 1) / S;
      if (ns > 0 && sample_pos(ns - 1, S) >= n) --ns;
    } else {
      ns = sample_load<kRowThreads>(row, n, sv);   // first: tau waits on these only
    }
  }
  // Two batches in flight: while one is compacted the next two are loading.
  // Loads past the row re-read its last position (the pass test drops them),
  // so no load sits behind a branch and the compiler waits only for the batch
  // it needs.
  auto load_batch = [&](float* v, int base) {
#pragma unroll
    for (int e = 0; e < kBatch; ++e) v[e] = row[min(base + e * kRowThreads + (int)threadIdx.x, n - 1)];
  };
  if constexpr (RANGES) {
    // Each wave streams its own contiguous range of the row (a multiple of 64
    // positions) and compacts its candidates into its own part of the LDS list
    // with ballots: no barrier until the row has been read.  The parts follow
    // each other in wave order, which is position order; after the select each
    // wave writes out its own part's share of the row.
    constexpr int NW = kRowThreads / 64, U = kBatch, kWaveCap = kRowCap / NW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int seg = (n + 64 * NW - 1) / (64 * NW) * 64;
    const int p0 = wave * seg, p1 = min(n, p0 + seg);
    // the row through a buffer that ends at the wave's range: a load past it
    // returns 0.0 and fetches nothing, so no load sits behind a branch and no
    // line is fetched twice
    const __amdgpu_buffer_rsrc_t rrs = wave_rsrc(row, p1 * 4);
    auto load_run = [&](float* v, int base) {
      const uint32_t voff = (uint32_t)(base + lane) * 4u;
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rrs, voff, 256 * u, 0));
    };
    float va[U], vb[U];
    load_run(va, p0);
    load_run(vb, p0 + 64 * U);
    const uint32_t tau = sampled ? sample_tau_near_max<kRowThreads>(sv, ns, n, k, hist, scratch) : 0u;
    uint32_t* wkey = ckey + wave * kWaveCap;
    Pos* wpos = cpos + wave * kWaveCap;
    uint32_t cnt = 0;                             // the wave's candidates so far (uniform)
    // With a positive threshold (the usual case) a key at or above it is a
    // float whose bits, read as a signed integer, are at or above the
    // threshold's without its sign bit (negative values and negative NaNs
    // fall below, positive NaNs above, as with keys): the pass compares the
    // raw bits and stores them, and they become keys only for the candidates,
    // after the pass.  The 0.0 read past the range fails that test, so only
    // the key test needs the position check.
    const bool raw = tau > 0x80000000u;           // uniform
    const int32_t tau_bits = (int32_t)(tau & 0x7fffffffu);
    auto run = [&](auto raw_bits, float* v, int base) {
      constexpr bool RAW = decltype(raw_bits)::value;
      uint32_t key[U];
      bool pass[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        key[u] = RAW ? __float_as_uint(v[u]) : order_key(v[u]);
        pass[u] = RAW ? (int32_t)key[u] >= tau_bits : base + 64 * u + lane < p1 && key[u] >= tau;
      }
      load_run(v, base + 2 * 64 * U);             // two runs ahead
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t mk = __ballot(pass[u]);
        // past the part's end every store lands on its last entry: the part
        // has overflowed and the row is selected whole, so nothing reads it
        const uint32_t at = min(cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u)),
                                (uint32_t)kWaveCap - 1u);
        if (pass[u]) {
          wkey[at] = key[u];
          wpos[at] = (Pos)(base + 64 * u + lane);
        }
        cnt += (uint32_t)__popcll(mk);
      }
    };
    auto pass_range = [&](auto raw_bits) {
      for (int base = p0; base < p1; base += 2 * 64 * U) {
        run(raw_bits, va, base);
        if (base + 64 * U < p1) run(raw_bits, vb, base + 64 * U);
      }
    };
    if (raw)
      pass_range(std::integral_constant<bool, true>());
    else
      pass_range(std::integral_constant<bool, false>());
    constexpr int R = kWaveCap / 64;
    __shared__ uint32_t wcnt[NW];
    __shared__ uint32_t wmax[NW];
    __shared__ uint32_t ecnt[2 * NW];
    if (raw) {
      // Each wave turns its part's raw bits into keys where they lie, takes
      // its largest key and pads the rest of the part with key 0, below the
      // (positive) threshold, which the select ignores: the parts need no
      // moving, and each wave writes out its own.
      uint32_t hi = 0u;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t i = (uint32_t)(64 * r + lane);
        const uint32_t x = i < cnt ? order_key(__uint_as_float(wkey[i])) : 0u;
        wkey[i] = x;
        hi = max(hi, x);
      }
      hi = wave_max(hi);
      if (lane == 0) wmax[wave] = hi;
    }
    if (lane == 0) wcnt[wave] = cnt;
    __syncthreads();
    uint32_t C = 0, before = 0;
    bool fits = true;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const uint32_t c = wcnt[v];
      fits = fits && c <= (uint32_t)kWaveCap;
      before += v < wave ? c : 0u;
      C += c;
    }
    if (!fits) C = kRowCap + 1;                   // a part overflowed: the whole row is selected
    const bool in_lds = fits && C >= (uint32_t)k; // uniform
    if (raw && in_lds) {
      // every candidate lies in [tau, the largest part maximum]
      uint32_t kmax = 0u;
#pragma unroll
      for (int v = 0; v < NW; ++v) kmax = max(kmax, wmax[v]);
      uint32_t take;
      const uint32_t kstar = select_kth_range<kRowThreads>(ckey, (uint32_t)kRowCap, (uint32_t)k, tau, kmax,
                                                           &take, hist, bucket, scratch);
      uint32_t key[R];
      int32_t pos[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        key[r] = wkey[64 * r + lane];
        pos[r] = (int32_t)wpos[64 * r + lane];
      }
      const uint32_t a0 = (uint32_t)(wave * kWaveCap);
      emit_runs<kRowThreads, R>(key, pos, a0, a0 + cnt, kstar, take, k, out, ecnt);
    } else if (in_lds) {                          // keys: move the parts together (all reads first)
      uint32_t rk[R];
      Pos rp[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t i = min((uint32_t)(64 * r + lane), cnt - (cnt > 0 ? 1u : 0u));
        rk[r] = wkey[i];
        rp[r] = wpos[i];
      }
      uint32_t hi = 0u;                           // the part's largest key
#pragma unroll
      for (int r = 0; r < R; ++r) hi = max(hi, cnt > 0 ? rk[r] : 0u);   // entries past cnt repeat the last one
      hi = wave_max(hi);
      if (lane == 0) wmax[wave] = hi;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t i = (uint32_t)(64 * r + lane);
        if (i < cnt) { ckey[before + i] = rk[r]; cpos[before + i] = rp[r]; }
      }
      __syncthreads();                            // the candidates, before the select reads them
      uint32_t kmax = 0u;
#pragma unroll
      for (int v = 0; v < NW; ++v) kmax = max(kmax, wmax[v]);
      uint32_t take;
      const uint32_t kstar = select_kth_range<kRowThreads>(ckey, C, (uint32_t)k, tau, kmax, &take, hist,
                                                           bucket, scratch);
      emit_by_waves<kRowThreads>(ckey, cpos, C, kstar, take, k, out, ecnt);
    } else {
      finish_row<kRowThreads>(row, n, k, C, kRowCap, ckey, cpos, out, hist, bucket, scratch);
    }
  } else {
    float va[kBatch], vb[kBatch];
    load_batch(va, 0);
    load_batch(vb, kStep);
    const uint32_t tau = sampled ? sample_tau<kRowThreads>(sv, ns, n, k, hist, scratch) : 0u;
    uint32_t C = 0;
    auto batch = [&](float* v, int base, uint32_t* tab) {
      uint32_t key[kBatch];
      bool pass[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        key[e] = order_key(v[e]);
        pass[e] = base + e * kRowThreads + (int)threadIdx.x < n && key[e] >= tau;
      }
      load_batch(v, base + 2 * kStep);            // two batches ahead
      C += compact_ordered<kRowThreads, kBatch>(key, pass, base, C, ckey, cpos, kRowCap, tab);
    };
    for (int base = 0; base < n; base += 2 * kStep) {
      batch(va, base, table[0]);
      if (base + kStep < n) batch(vb, base + kStep, table[1]);
    }
    __syncthreads();                              // the compacted candidates, before the select reads them
    finish_row<kRowThreads>(row, n, k, C, kRowCap, ckey, cpos, out, hist, bucket, scratch);
  }
}

// ---------------------------------------------------------- long rows --

template <int kChunk>
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float* __restrict__ logits,
                                                               int64_t ld, BatchArgs b, int k,
                                                               TopkWorkspace ws,
                                                               int32_t* __restrict__ topk,
                                                               int64_t ldo) {
  constexpr int kPer = kChunk / kThreads;
  const int t = blockIdx.y;
  const int c = blockIdx.x;
  const int n = token_pos_wave(b, t).n;
  if (n <= k) {
    if (c == 0) write_all<kThreads>(topk + (size_t)t * ldo, n, k);
    return;
  }
  const int s0 = c * kChunk;
  if (s0 >= n) {                                // past the row: an empty slot
    if (threadIdx.x == 0) ws.counts[(size_t)t * ws.nslots + c] = 0u;
    return;
  }
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t table[kPer * kThreads / 64];
  __shared__ uint32_t scratch[scratch_words<kThreads>()];
  const float* row = logits + (size_t)t * ld;
  const bool sampled = n > 4 * k;               // else every position is a candidate
  float sv[sample_per<kThreads>()];
  int ns = 0;
  if (sampled)                                  // first: tau waits on these only
    ns = ws.samp ? sample_load_compact<kThreads>(ws.samp + (size_t)t * kMaxSample, n, sv)
                 : sample_load<kThreads>(row, n, sv);
  float v[kPer];                                // the chunk's loads fly while tau is placed
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int s = s0 + e * kThreads + threadIdx.x;
    v[e] = s < n ? row[s] : 0.f;
  }
  const uint32_t tau = sampled ? sample_tau<kThreads>(sv, ns, n, k, hist, scratch) : 0u;
  uint32_t key[kPer];
  bool pass[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    key[e] = order_key(v[e]);
    pass[e] = s0 + e * kThreads + (int)threadIdx.x < n && key[e] >= tau;
  }
  const size_t slot = ((size_t)t * ws.nslots + c) * ws.slot_cap;
  const uint32_t cnt = compact_ordered<kThreads, kPer>(key, pass, s0, 0, ws.cand_key + slot,
                                                       ws.cand_pos + slot, kChunk, table);
  if (threadIdx.x == 0) ws.counts[(size_t)t * ws.nslots + c] = cnt;
}

#ifndef IDX_RESOLVE_THREADS
#define IDX_RESOLVE_THREADS 1024
#endif
constexpr int kResolveThreads = IDX_RESOLVE_THREADS;
constexpr int kSpecSlots = 128;     // rows of up to 128 filter slots preload their candidates
constexpr int kSpecPer = 8;         // entries each resolve thread preloads

// One work-group per long row: gathers the row's candidate slots in order and
// finishes the row.  Works for either slot layout of the workspace.
__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(
    const float* __restrict__ logits, int64_t ld, BatchArgs b, int k, TopkWorkspace ws,
    int32_t* __restrict__ topk, int64_t ldo) {
  constexpr int NT = kResolveThreads;
  const int t = blockIdx.x;
  const int n = token_pos_wave(b, t).n;
  int32_t* out = topk + (size_t)t * ldo;
  if (n <= k) {
    write_all<NT>(out, n, k);
    return;
  }
  __shared__ uint32_t ckey[kCandCap];
  __shared__ int32_t cpos[kCandCap];
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t pre[kMaxSlots + 1];
  __shared__ uint32_t bucket[64];
  __shared__ uint32_t scratch[scratch_words<NT>()];
  __shared__ uint32_t krange[2];
  if (threadIdx.x == 0) { krange[0] = 0xffffffffu; krange[1] = 0u; }   // before the scan's barriers
  const int nsl = min(ws.nslots, kMaxSlots);
  const uint32_t* cnts = ws.counts + (size_t)t * ws.nslots;
  const uint32_t cap = (uint32_t)ws.slot_cap;
  const size_t base = (size_t)t * ws.nslots * ws.slot_cap;
  // With at most kSpecSlots slots, each slot's first entries are loaded before
  // the counts are known (NT / nsl threads per slot, kSpecPer entries each),
  // so the count and candidate round trips overlap.
  const bool spec = nsl <= kSpecSlots && nsl > 0;
  const int tps = spec ? NT / nsl : 1;
  const int my_slot = spec ? min((int)threadIdx.x / tps, nsl - 1) : 0;
  const int my_lane = spec ? (int)threadIdx.x - my_slot * tps : 0;
  const bool my_ok = spec && (int)threadIdx.x < tps * nsl;
  uint32_t sk[kSpecPer];
  int32_t sp[kSpecPer];
  if (spec) {
    const size_t sb = base + (size_t)my_slot * ws.slot_cap;
#pragma unroll
    for (int u = 0; u < kSpecPer; ++u) {
      const uint32_t j = min((uint32_t)(my_lane + tps * u), cap - 1u);
      sk[u] = ws.cand_key[sb + j];
      sp[u] = ws.cand_pos[sb + j];
    }
  }
  // slot offsets (every slot count is written; clamp anyway): one wave scans
  // up to 64 slots, the block scans more
  if (nsl <= 64) {
    if (threadIdx.x < 64) {
      const int c = threadIdx.x;
      const uint32_t v = c < nsl ? min(cnts[c], cap) : 0u;
      const uint32_t incl = wave_sum_incl(v);
      if (c < nsl) pre[c] = incl - v;
      if (c == 63) pre[nsl] = incl;
    }
  } else {
    const int per = (nsl + NT - 1) / NT;
    const int c0 = min(nsl, per * (int)threadIdx.x), c1 = min(nsl, c0 + per);
    uint32_t s = 0;
    for (int c = c0; c < c1; ++c) s += min(cnts[c], cap);
    uint32_t total;
    uint32_t run = block_scan_excl<NT>(s, &total, scratch);
    for (int c = c0; c < c1; ++c) { pre[c] = run; run += min(cnts[c], cap); }
    if (threadIdx.x == 0) pre[nsl] = total;
  }
  __syncthreads();
  const uint32_t C = pre[nsl];
  const float* row = logits + (size_t)t * ld;
  auto at = [&](uint32_t i) {                   // workspace index of candidate i (position order)
    int lo = 0, hi = nsl - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return base + (size_t)lo * ws.slot_cap + (i - pre[lo]);
  };
  if (C >= (uint32_t)k && C <= (uint32_t)kCandCap) {
    uint32_t lo = 0xffffffffu, hi = 0u;         // the keys' range, taken on the way into LDS
    auto put = [&](uint32_t i, uint32_t key, int32_t pos) {
      ckey[i] = key;
      cpos[i] = pos;
      lo = min(lo, key);
      hi = max(hi, key);
    };
    if (spec) {
      const uint32_t cnt = pre[my_slot + 1] - pre[my_slot], at0 = pre[my_slot];
      if (my_ok) {
#pragma unroll
        for (int u = 0; u < kSpecPer; ++u) {
          const uint32_t j = (uint32_t)(my_lane + tps * u);
          if (j < cnt) put(at0 + j, sk[u], sp[u]);
        }
        // entries beyond the preloaded ones (rare): read them now
        const size_t sb = base + (size_t)my_slot * ws.slot_cap;
        for (uint32_t j = (uint32_t)(my_lane + tps * kSpecPer); j < cnt; j += (uint32_t)tps)
          put(at0 + j, ws.cand_key[sb + j], ws.cand_pos[sb + j]);
      }
    } else {
      for (uint32_t i = threadIdx.x; i < C; i += NT) {
        const size_t a = at(i);
        put(i, ws.cand_key[a], ws.cand_pos[a]);
      }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((threadIdx.x & 63) == 0) { atomicMin(&krange[0], lo); atomicMax(&krange[1], hi); }
    __syncthreads();
    uint32_t take;
    const uint32_t kstar = select_kth_range<NT>(ckey, C, (uint32_t)k, krange[0], krange[1], &take,
                                                hist, bucket, scratch);
    emit_ordered<NT>([&](uint32_t i) { return make_uint2(ckey[i], (uint32_t)cpos[i]); }, C, kstar,
                     take, k, out, scratch);
  } else if (C > (uint32_t)kCandCap) {          // too many for LDS: read the slots in place
    uint32_t take;
    const uint32_t kstar = radix_kth<NT, 3>([&](auto&& fn) {
      for (int c = 0; c < nsl; ++c) {
        const size_t sb = base + (size_t)c * ws.slot_cap;
        for (uint32_t i = threadIdx.x; i < pre[c + 1] - pre[c]; i += NT) fn(ws.cand_key[sb + i]);
      }
    }, (uint32_t)k, &take, hist, scratch);
    emit_ordered<NT>([&](uint32_t i) {
      const size_t a = at(i);
      return make_uint2(ws.cand_key[a], (uint32_t)ws.cand_pos[a]);
    }, C, kstar, take, k, out, scratch);
  } else {
    finish_row<NT>(row, n, k, C, kCandCap, ckey, cpos, out, hist, bucket, scratch);   // fewer than k: whole row
  }
}

}  // namespace

bool topk_uses_long_rows(int64_t T, int max_seq_len) { return T < 256 && max_seq_len > 8192; }

int topk_chunk(bool sample_copy) { return sample_copy ? kChunkSampled : kChunkPlain; }

int topk_nchunks(int max_seq_len, bool sample_copy) {
  const int c = topk_chunk(sample_copy);
  return (max_seq_len + c - 1) / c;
}

int topk_max_seq_len() { return kMaxLongRow; }

hipError_t launch_topk_resolve(const float* logits, int64_t ld, const BatchArgs& b,
                               const TopkWorkspace& ws, int k, int32_t* out, int64_t ldo,
                               hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  IDX_LAUNCH("topk_resolve_kernel", (topk_resolve_kernel), dim3((unsigned)b.num_tokens),
             dim3(kResolveThreads), stream, logits, ld, b, k, ws, out, ldo);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t ld, const BatchArgs& b, const TopkWorkspace& ws,
                       int k, int32_t* out, int64_t ldo, hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  if (topk_uses_long_rows(b.num_tokens, b.max_seq_len)) {
    // the workspace layout fixed the chunking: one slot of slot_cap entries per chunk
    const dim3 grid((unsigned)std::max(1, ws.nslots), (unsigned)b.num_tokens);
    if (ws.slot_cap == kChunkSampled)
      IDX_LAUNCH("topk_filter_kernel", (topk_filter_kernel<kChunkSampled>), grid, dim3(kThreads),
                 stream, logits, ld, b, k, ws, out, ldo);
    else if (ws.slot_cap == kChunkPlain)
      IDX_LAUNCH("topk_filter_kernel", (topk_filter_kernel<kChunkPlain>), grid, dim3(kThreads),
                 stream, logits, ld, b, k, ws, out, ldo);
    else
      return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk_resolve(logits, ld, b, ws, k, out, ldo, stream);
  } else {
    // rows whose sample the scoring kernel copied out are read once, each wave
    // its own range; rows whose sample is gathered first keep the interleaved
    // pass (faster there: the gather has just touched every line of the row)
    const bool small = b.max_seq_len <= 65536;
    if (small && ws.samp != nullptr)
      IDX_LAUNCH("topk_rows_kernel", (topk_rows_kernel<uint16_t, true>), dim3((unsigned)b.num_tokens),
                 dim3(kRowThreads), stream, logits, ld, b, k, out, ldo, ws.samp);
    else if (small)
      IDX_LAUNCH("topk_rows_kernel", (topk_rows_kernel<uint16_t, false>), dim3((unsigned)b.num_tokens),
                 dim3(kRowThreads), stream, logits, ld, b, k, out, ldo, ws.samp);
    else if (ws.samp != nullptr)
      IDX_LAUNCH("topk_rows_kernel", (topk_rows_kernel<int32_t, true>), dim3((unsigned)b.num_tokens),
                 dim3(kRowThreads), stream, logits, ld, b, k, out, ldo, ws.samp);
    else
      IDX_LAUNCH("topk_rows_kernel", (topk_rows_kernel<int32_t, false>), dim3((unsigned)b.num_tokens),
                 dim3(kRowThreads), stream, logits, ld, b, k, out, ldo, ws.samp);
  }
  return hipGetLastError();
}

}  // namespace idx

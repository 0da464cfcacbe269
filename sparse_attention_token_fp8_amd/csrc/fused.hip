// Fused score + top-k for batches scored one token per work-group (decode
// batches over long contexts): the scores never reach HBM.
//
// IndexCache blog post, SparseAttnIndexer.forward_cuda and the op body: one op
// takes q_fp8, the paged K cache and the folded weights and leaves the top-k
// positions in topk_indices_buffer; no score tensor crosses its boundary.
//
// Method.  A row of n causal positions is scored by work-groups that each own
// a chunk of consecutive blocks (about one chunk per CU over the batch; the
// chunk's eight waves take its blocks one at a time).
//  1. Each work-group keeps its chunk's scores in LDS.  It places a threshold
//     tau_c with at least m_c keys of the chunk at or above it, where m_c is
//     the chunk's expected share of the row's top k plus a wide margin
//     (chunk_keep), and compacts the keys >= tau_c, in position order, into the
//     chunk's slot of the workspace, with tau_c and the count beside them.
//     (A chunk with at most m_c positions keeps them all, tau_c = 0.)
//  2. One work-group per row gathers the slots.  Let T = max_c tau_c.  Every
//     key of the row at or above T is a candidate (a chunk drops only keys
//     below its tau_c <= T).  So if at least k candidates are >= T, the k-th
//     largest key of the row is the k-th largest candidate, every key above it
//     and every key equal to it is a candidate, and the exact select over the
//     candidates (ties to the lower position) is the exact top-k of the row.
//  3. Otherwise (some chunk held far more than its share of the row's top k)
//     the row is scored again, whole, and selected from all its keys.  So the
//     result never depends on the thresholds; they only decide how much work
//     the exact select does.
//
// The rescoring uses the same per-block operation sequence as the scoring
// kernels, so every key equals the one idx_logits would produce, and the rows
// equal those of idx_logits + idx_topk bit for bit.

#include "common.hpp"
#include "launch.hpp"
#include "score_device.hpp"
#include "topk_device.hpp"
#include "fp4_device.hpp"


#include <algorithm>
#include <type_traits>

namespace idx {
namespace {


// Keys a chunk of `nvalid` of a row's n positions keeps at least: its expected
// share e of the row's top k plus 6 sqrt(e) + 8.  The number of top-k keys in
// a chunk is hypergeometric with variance below e, so with scores that do not
// depend on the position a chunk holds more than that with probability below
// 1e-10 (for 8 rows x 131072 positions, k = 2048: 7e-11 per chunk, about
// 3e-8 per call); and where it does happen the row is rescored (step 3).
__device__ __forceinline__ uint32_t chunk_keep(int k, int nvalid, int n) {
  const float e = (float)k * (float)nvalid / (float)n;
  return (uint32_t)ceilf(e + 6.f * sqrtf(e)) + 8u;
}

// Threshold histogram: the top 12 bits of the order key (sign, exponent and
// three mantissa bits, so bins are an eighth of an octave wide), counted by
// the scoring loop.
constexpr int kTauBins = 4096;
constexpr int kTauShift = 20;

// In the histogram h[0..64*PER) of one work-group, the bin holding the
// need-th largest entry (1 <= need <= total), found by one wave on its own:
// lane i sums bins [(63-i)*PER, (64-i)*PER) (lanes in descending key order),
// one scan finds the lane whose bins reach `need`, a second scan over that
// lane's bins the bin.  *above = entries in higher bins.
template <int PER>
__device__ __forceinline__ uint32_t wave_find_bin(const uint32_t* h, uint32_t need, uint32_t* above,
                                                  int lane) {
  static_assert(PER % 4 == 0 && PER <= 64, "bins per lane");
  constexpr int NB = 64 * PER, Q = PER / 4;
  const uint32_t* hb = h + NB - PER * (lane + 1);
  // Lanes' ranges are PER words apart, so at the same offset they would all hit
  // one bank group: lane l reads its 16-byte chunks starting at chunk l % Q.
  uint32_t sum = 0u;
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(hb + 4 * ((i + lane) % Q));
    sum += v.x + v.y + v.z + v.w;
  }
  const uint32_t incl = wave_sum_incl(sum);
  const int L = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;
  const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
  const uint32_t* hl = h + NB - PER * (L + 1);
  const uint32_t c = lane < PER ? hl[PER - 1 - lane] : 0u;   // lane j: the lane's j-th highest bin
  const uint32_t inc2 = wave_sum_incl(c);
  const int j = __ffsll((unsigned long long)__ballot(lane < PER && before + inc2 >= need)) - 1;
  *above = before + (uint32_t)__builtin_amdgcn_readlane((int)(inc2 - c), j);
  return (uint32_t)(NB - PER * (L + 1) + (PER - 1 - j));
}

// Step 1, after the work-group's scores are in `kept` (position order), their
// histogram in `hist` and their largest key in table[0], every wave past the
// scoring loop.  tau is the lower edge of the bin holding the m-th largest key
// (so at least m keys are >= tau, and at most the bin's other keys besides
// them); every wave finds it on its own from the shared histogram.  NT threads, NT >= 256, for chunks of up to MAXPOS
// positions; `table` holds 65 words, 129 when MAXPOS / 64 > 64.
template <int NT, int MAXPOS>
__device__ __forceinline__ void chunk_filter(const float* kept, int t, int cx, int chunk_blocks,
                                             int n, int k, const KeepSlots& ks, uint32_t* hist,
                                             uint32_t* table) {
  constexpr int E = MAXPOS / NT;
  const int lane = threadIdx.x & 63;
  const int base = cx * chunk_blocks * kBlock;
  const int nvalid = min(n - base, chunk_blocks * kBlock);
  const uint32_t m = chunk_keep(k, nvalid, n);
  const bool cut = (uint32_t)nvalid > m;          // else the chunk keeps every key
  uint32_t key[E];
  bool pass[E];
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = kept[e * NT + threadIdx.x];   // all reads first (in bounds)
  const uint32_t kmax = table[0];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    pass[e] = e * NT + (int)threadIdx.x < nvalid;
    key[e] = pass[e] ? order_key(v[e]) : 0u;
  }
  uint32_t tau = 0u;
  if (cut) {                                      // uniform over the work-group
    uint32_t above;
    tau = wave_find_bin<kTauBins / 64>(hist, m, &above, lane) << kTauShift;
#pragma unroll
    for (int e = 0; e < E; ++e) pass[e] = pass[e] && key[e] >= tau;
  }
  const size_t slot = (size_t)t * ks.nslots + cx;
  uint2* dst = ks.cand + slot * ks.cap;
  const uint32_t cap = (uint32_t)ks.cap;
  auto put = [&](uint32_t i, uint32_t kk, int pos) {
    if (i < cap) dst[i] = make_uint2(kk, (uint32_t)pos);
  };
  uint32_t cnt;
  if constexpr (E * (NT / 64) <= 64) {
    cnt = compact_ordered_to<NT, E>(key, pass, base, 0u, table + 1, put);
  } else {                                      // two halves in position order, own count tables
    constexpr int H = E / 2;
    const uint32_t c1 = compact_ordered_to<NT, H>(key, pass, base, 0u, table + 1, put);
    cnt = c1 + compact_ordered_to<NT, H>(key + H, pass + H, base + H * NT, c1, table + 65, put);
  }
  if (threadIdx.x == 0) {
    ks.counts[slot] = cnt;
    ks.taus[slot] = tau;
    ks.maxes[slot] = kmax;
  }
}

// ---------------------------------------------------------- scoring --
// Step 1 by one work-group of kDynWaves waves per CU, whose waves take the
// chunk's blocks one at a time from a work-group counter: no CU holds two
// work-groups of which the younger is served later and ends last, waves that
// the SIMDs serve faster take more blocks, and the chunk's threshold and
// compaction run once per CU.
constexpr int kDynWaves = 8;
constexpr int kDynThreads = 64 * kDynWaves;
constexpr int kDynMaxBlocks = 128;              // a chunk's blocks: two block ids per lane

// Scores one token's chunk (up to kDynMaxBlocks blocks): position s of the
// chunk's scores goes to kept[s - its first position] (LDS), its order key is
// counted in khist[key >> kTauShift] (LDS, zeroed before the call) and the
// largest key is accumulated in *khi; *next is the LDS block counter, set to
// kDynWaves * (NB - 1) before the call (each wave's first NB - 1 blocks are
// wave, wave + kDynWaves, ...).  With FK every wave quantises the chunk's new
// rows, the wave that scores a row's block patches it into its staged copy,
// and wave 0 writes the token's own row to the cache.  Returns the token's
// causal count n, or -1 when the chunk holds none of its positions.
// FP4: the cache is the FP4 one, its blocks loaded straight into the MFMA
// layout as fp4_decode_body does (`lds`: kLinScratch per wave); else each
// block passes through the wave's LDS slot (`lds`: kBlockBytes per wave).
template <int NB, bool FK, bool FP4>
__device__ __forceinline__ int dyn_body(int cx, int t, const uint8_t* __restrict__ q8,
                                        const float* __restrict__ w, const CacheArgs& cache,
                                        const BatchArgs& b, int chunk_blocks, bool ident,
                                        uint8_t* lds, const NewRows& nk, float* kept,
                                        uint32_t* khist, uint32_t* khi, uint32_t* next) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lb0 = cx * chunk_blocks;
  int bt_full[2] = {-1, -1};                    // raw ids; checked only once they are needed
  if (ident) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (lane + 64 * h < chunk_blocks)
        bt_full[h] = b.bt[(int64_t)t * b.bt_stride + min(lb0 + lane + 64 * h, (int)b.bt_stride - 1)];
  }
  TokenPos tp;
  if (ident) {                                  // one new token per request: token t is request t
    tp.r = t;
    tp.q0 = t;
    tp.nq = 1;
    tp.len = b.seq_lens[t];
    tp.n = min(max(tp.len, 0), b.max_seq_len);
  } else {
    tp = token_pos_wave(b, t);
  }
  QFrag f[1];
  load_q(f[0], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
  const int n = tp.n;
  if (lb0 * kBlock >= n) return -1;
  const int nblk = min(chunk_blocks, (n - lb0 * kBlock + kBlock - 1) / kBlock);
  const int lp = lane_pos(lane);
  uint32_t hi = 0u;                             // largest key of this lane
  auto emit = [&](int j, float v) {             // j: the chunk's block, < nblk
    const int s = (lb0 + j) * kBlock + lp;
    if (s < n) {
      kept[s - lb0 * kBlock] = v;
      const uint32_t key = order_key(v);
      atomicAdd(&khist[key >> kTauShift], 1u);
      hi = max(hi, key);
    }
  };
  auto keep_max = [&]() {
    const uint32_t m = wave_max(hi);
    if (lane == 0) atomicMax(khi, m);
  };
  if (cache.num_blocks == 0) {                  // no K at all: every score is 0
    for (int j = wave; j < nblk; j += kDynWaves) emit(j, 0.f);
    keep_max();
    return n;
  }
  // lane j holds the physical blocks of the chunk's blocks j and 64 + j
  int pbl[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    if (ident && nblk == chunk_blocks)
      pbl[h] = (j < chunk_blocks && lb0 + j < b.bt_stride && bt_full[h] >= 0 &&
                bt_full[h] < cache.num_blocks) ? bt_full[h] : -1;
    else
      pbl[h] = j < nblk ? (int)phys_block(b, cache, tp.r, lb0 + j) : -1;
  }
  auto pblock = [&](int j) {                    // j uniform, < kDynMaxBlocks
    return __builtin_amdgcn_readlane(j < 64 ? pbl[0] : pbl[1], j & 63);
  };
  using Ring = std::conditional_t<FP4, KBlock4, WaveStage>;
  // block j of the chunk (uniform); from nblk on it loads nothing
  auto stage = [&](Ring& st, int j) {
    const int pb = pblock(min(j, kDynMaxBlocks - 1));
    if constexpr (FP4)
      fp4_block_load<kLoadStream>(st, cache.data + (int64_t)max(pb, 0) * kFp4BlockBytes,
                                  (j < nblk && pb >= 0) ? kFp4BlockBytes : 0, lane);
    else
      wave_stage_load(st, cache.data + (int64_t)max(pb, 0) * kBlockBytes,
                      (j < nblk && pb >= 0) ? kBlockBytes : 0, lane);
  };
  auto grab = [&]() {
    uint32_t j = 0u;
    if (lane == 0) j = atomicAdd(next, 1u);
    return __builtin_amdgcn_readfirstlane((int)j);
  };
  uint8_t* slot = lds + wave * (FP4 ? kLinScratch : kBlockBytes);
  int jr[NB];                                   // the block each ring entry holds
  Ring ring[NB];
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    jr[u] = wave + u * kDynWaves;
    stage(ring[u], jr[u]);
  }
  LinFrag lf;
  make_lin<1>(lf, f, slot, lane);

  // FP8: a row is 32 lanes' 4-byte codes and a 4-byte scale (all ones: leave
  // the row as the cache has it); FP4: each group's 16 code bytes and its
  // exponent byte (all ones: leave it).
  uint32_t fcode[kMaxFusedRows];
  uint4 fcode4[kMaxFusedRows];
  uint32_t fscale[kMaxFusedRows];
  int fpos0 = 0, nfix = 0;
  if (FK) {                                     // the chunk's new rows, as decode_body
    const int newlo = tp.len - tp.nq;
    const int lo = max(newlo, lb0 * kBlock);
    const int hi2 = min(n - 1, (lb0 + nblk) * kBlock - 1);
    nfix = min(kMaxFusedRows, max(0, hi2 - lo + 1));
    fpos0 = lo;
#pragma unroll
    for (int i = 0; i < kMaxFusedRows; ++i) {
      fcode[i] = 0u;
      fcode4[i] = make_uint4(0u, 0u, 0u, 0u);
      fscale[i] = 0xFFFFFFFFu;
      if (i < nfix) {
        const int P = lo + i;
        const int row = tp.q0 + (P - newlo);
        const int64_t want = nk.slots[row];
        const int pb = pblock(P / kBlock - lb0);
        const bool patch = pb >= 0 && want == (int64_t)pb * kBlock + P % kBlock;
        const bool own = wave == 0 && row == t && want >= 0 && want < nk.num_slots;
        if constexpr (FP4) {
          int e;
          fcode4[i] = fp4_quant_group(nk.k + (int64_t)row * nk.stride + 32 * (lane >> 4), &e);
          if (patch) fscale[i] = (uint32_t)(e + 127);
          if (own) fp4_write_row(nk.cache, want, fcode4[i], e, lane);
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(nk.k + (int64_t)row * nk.stride + (lane & 31) * 4);
          int e;
          const uint32_t code = quant_row_lane(v, &e);
          const uint32_t sc = __float_as_uint(pow2f(e));
          fcode[i] = code;
          if (patch) fscale[i] = sc;
          if (own) {
            uint8_t* cb = nk.cache + (want / kBlock) * kBlockBytes;
            if (lane < 32) *reinterpret_cast<uint32_t*>(cb + (want % kBlock) * kHeadDim + lane * 4) = code;
            if (lane == 0) *reinterpret_cast<uint32_t*>(cb + kCodeBytes + (want % kBlock) * 4) = sc;
          }
        }
      }
    }
  }

  // Each step takes the next block for the ring entry just consumed, then
  // scores the oldest entry; a wave stops at its first block past the chunk
  // (the counter only grows, so every later one is past it too).
  for (;;) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int s = (u + NB - 1) % NB;
      jr[s] = grab();
      stage(ring[s], jr[s]);
      __builtin_amdgcn_sched_barrier(0);
      const int j = jr[u];
      if (j >= nblk) {
        keep_max();
        return n;
      }
      float v;
      if constexpr (FP4) {
        KBlock4& kb = ring[u];
        if (FK) {
#pragma unroll
          for (int i = 0; i < kMaxFusedRows; ++i) {
            const int P = fpos0 + i;
            if (i < nfix && fscale[i] != 0xFFFFFFFFu && P / kBlock == lb0 + j)
              fp4_patch_row(kb, P % kBlock, fcode4[i], fscale[i], lane);
          }
        }
        fp4_block_scores<1>(f, lf, kb, &v);
      } else {
        wave_stage_store(ring[u], slot, lane);
        if (FK) {
#pragma unroll
          for (int i = 0; i < kMaxFusedRows; ++i) {
            const int P = fpos0 + i;
            if (i < nfix && fscale[i] != 0xFFFFFFFFu && P / kBlock == lb0 + j) {
              const int rr = P % kBlock;
              if (lane < 32)
                *reinterpret_cast<uint32_t*>(slot + rr * kHeadDim + (((lane >> 2) ^ (rr & 7)) << 4) +
                                             (lane & 3) * 4) = fcode[i];
              if (lane == 0) *reinterpret_cast<uint32_t*>(slot + kCodeBytes + rr * 4) = fscale[i];
            }
          }
        }
        wave_sync_lds();
        KBlock kb;
        lds_kblock(kb, slot, lane);
        wave_sync_lds();                        // reads done before the slot is rewritten
        block_scores<1>(f, lf, kb, &v);
      }
      emit(j, v);
    }
  }
}

#ifndef IDX_DYN_RING
#define IDX_DYN_RING 2
#endif
// MAXB: the largest chunk it takes (64 or kDynMaxBlocks blocks), which sizes
// `kept` and the filter's registers.  FP4: the FP4 cache.
template <int NB, bool FK, int MAXB, bool FP4>
__global__ __launch_bounds__(kDynThreads) void score_keep_dyn_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    int chunk_blocks, int ident, NewRows nk, int k, KeepSlots ks) {
  static_assert(MAXB <= kDynMaxBlocks, "two block ids per lane");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDynWaves * (FP4 ? kLinScratch : kBlockBytes)];
  __shared__ float kept[MAXB * kBlock];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kTauBins];
  __shared__ uint32_t table[1 + MAXB];
  __shared__ uint32_t next;
  for (int i = threadIdx.x; i < kTauBins / 4; i += kDynThreads)
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) {
    table[0] = 0u;
    next = (uint32_t)(kDynWaves * (NB - 1));
  }
  __syncthreads();
  int cx, ry;
  xcd_spread(&cx, &ry);
  const int n = dyn_body<NB, FK, FP4>(cx, ry, q8, w, cache, b, chunk_blocks, ident != 0, lds, nk,
                                      kept, hist, table, &next);
  if (n <= k) return;                           // nothing here, or a row the resolve takes whole
  __syncthreads();                              // every wave's scores are in `kept`
  chunk_filter<kDynThreads, MAXB * kBlock>(kept, ry, cx, chunk_blocks, n, k, ks, hist, table);
}

// ------------------------------------------------------------- resolve --

#ifndef IDX_RES_THREADS
#define IDX_RES_THREADS 1024
#endif
constexpr int kResThreads = IDX_RES_THREADS;
constexpr int kResCap = 8192;                   // candidates a row can hold in LDS
constexpr int kRescoreWaves = kResThreads / 64 < 8 ? kResThreads / 64 : 8;
constexpr int kSpecSlots = 128;                 // rows of up to 128 slots preload candidates
constexpr int kSpecPer = 8192 / kResThreads;    // entries each thread preloads

struct ResolveLds {
  uint32_t ckey[kResCap];
  int32_t cpos[kResCap];
  uint32_t hist[kBins1];
  uint32_t pre[kMaxSlots + 1];
  uint32_t bucket[64];
  uint32_t scratch[scratch_words<kResThreads>()];
  uint32_t emit[2 * (kResThreads / 64)];        // per-wave counts of the row's writer
  uint32_t misc[4];                             // T, largest key, in-place count or K*, bucket fill or take
};
struct RescoreLds {
  uint8_t stage[kRescoreWaves][kBlockBytes];
  uint8_t lin[kRescoreWaves][kLinScratch];
};
constexpr size_t kResolveSmem = sizeof(ResolveLds) > sizeof(RescoreLds) ? sizeof(ResolveLds)
                                                                         : sizeof(RescoreLds);

// Step 3: keys of all n positions of token t's row into keys[0..n), by
// kRescoreWaves waves of the work-group (the others idle), with the scoring
// kernels' per-block operations.
template <bool FP4>
__device__ __forceinline__ void rescore_row(const uint8_t* __restrict__ q8,
                                            const float* __restrict__ w, const CacheArgs& cache,
                                            const BatchArgs& b, int t, int r, int n,
                                            uint32_t* __restrict__ keys, RescoreLds* sm) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (wave >= kRescoreWaves) return;
  QFrag f[1];
  load_q(f[0], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
  LinFrag lf;
  make_lin<1>(lf, f, sm->lin[wave], lane);
  uint8_t* slot = sm->stage[wave];
  const int lp = lane_pos(lane);
  const int nb = (n + kBlock - 1) / kBlock;
  for (int lb = wave; lb < nb; lb += kRescoreWaves) {
    const int64_t pb = phys_block(b, cache, r, lb);
    if constexpr (FP4) {
      KBlock4 kb;
      fp4_block_load<kLoadStream>(kb, cache.data + (pb >= 0 ? pb : 0) * kFp4BlockBytes,
                                  pb >= 0 ? kFp4BlockBytes : 0, lane);
      float v;
      fp4_block_scores<1>(f, lf, kb, &v);
      const int s = lb * kBlock + lp;
      if (s < n) keys[s] = order_key(v);
      continue;
    }
    WaveStage st;
    wave_stage_load(st, cache.data + (pb >= 0 ? pb : 0) * kBlockBytes, pb >= 0 ? kBlockBytes : 0,
                    lane);
    wave_stage_store(st, slot, lane);
    wave_sync_lds();
    KBlock kb;
    lds_kblock(kb, slot, lane);
    wave_sync_lds();                            // reads done before the slot is rewritten
    float v;
    block_scores<1>(f, lf, kb, &v);
    const int s = lb * kBlock + lp;
    if (s < n) keys[s] = order_key(v);
  }
}

// A wave's run of the row's candidates, held in registers: wave w owns
// candidates [w R, (w+1) R) of ckey/cpos[0..C) (ascending position order),
// R a multiple of 64 and at most 64 E, lane l entries l, l + 64, ...
template <int NT>
struct RowRun {
  static constexpr int E = kResCap / NT;
  uint32_t key[E];
  int32_t pos[E];
  uint32_t a0, a1;                              // the run, clipped to C
  int ne;                                       // iterations holding any of it
  __device__ __forceinline__ void load(const uint32_t* ckey, const int32_t* cpos, uint32_t C) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const uint32_t R = (C + 64 * NW - 1) / (64 * NW) * 64;
    a0 = min(C, wave * R);
    a1 = min(C, a0 + R);
    ne = (int)((a1 - a0 + 63u) / 64u);
#pragma unroll
    for (int e = 0; e < E; ++e) {               // every read issued together (in bounds)
      const uint32_t j = min(a0 + 64u * e + lane, C - 1u);
      key[e] = ckey[j];
      pos[e] = cpos[j];
    }
  }
  __device__ __forceinline__ bool valid(int e) const {
    return a0 + 64u * e + (threadIdx.x & 63) < a1;
  }
};

// The row's k entries from the candidates of every wave's run (emit_runs).
template <int NT>
__device__ __forceinline__ void emit_row_waves(const RowRun<NT>& run, uint32_t kstar,
                                               uint32_t take_eq, int k, int32_t* __restrict__ out,
                                               uint32_t* counts) {
  emit_runs<NT, RowRun<NT>::E>(run.key, run.pos, run.a0, run.a1, kstar, take_eq, k, out, counts);
}

// Steps 2 and 3 for one row per work-group.  The row's length, the slot
// counts, thresholds and maxima and (for rows of up to kSpecSlots slots) the
// first entries of every slot are loaded at once, so the gather costs one
// round trip to memory.
template <bool FP4>
__global__ __launch_bounds__(kResThreads) void topk_keep_resolve_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    int ident, int k, KeepSlots ks, int32_t* __restrict__ topk, int64_t ldo) {
  constexpr int NT = kResThreads;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kResolveSmem];
  ResolveLds* sm = reinterpret_cast<ResolveLds*>(smem);
  const int t = blockIdx.x;
  const uint32_t cap = (uint32_t)ks.cap;
  const size_t rbase = (size_t)t * ks.nslots;   // the row's first slot
  // Preload, before the row's length is known: thread i takes slot i / tps of
  // the kSpecSlots (or fewer) first slots; entries past a slot's count are
  // read but never used.
  const int nsp = min(ks.nslots, kSpecSlots);
  const int tps = NT / nsp;
  const int my_slot = min((int)threadIdx.x / tps, nsp - 1);
  const int my_lane = (int)threadIdx.x - my_slot * tps;
  const bool my_ok = (int)threadIdx.x < tps * nsp;
  uint2 sc[kSpecPer];
  {
    const size_t sb = (rbase + my_slot) * cap;
#pragma unroll
    for (int u = 0; u < kSpecPer; ++u) sc[u] = ks.cand[sb + min((uint32_t)(my_lane + tps * u), cap - 1u)];
  }
  // Slot summaries of the first 64 slots (lane c of every wave reads slot c;
  // wave 0 uses them) and, for one token per request, the row's length: all
  // issued with the preload, unconditionally, so the row costs one round trip.
  const int c0 = min((int)threadIdx.x & 63, ks.nslots - 1);
  const uint32_t v0 = ks.counts[rbase + c0];
  const uint32_t tv0 = ks.taus[rbase + c0];
  const uint32_t mx0 = ks.maxes[rbase + c0];
  const int len_t = b.seq_lens[min(t, b.num_reqs - 1)];
  int r, n;
  if (ident) {                                  // one new token per request: token t is request t
    r = t;
    n = min(max(len_t, 0), b.max_seq_len);
  } else {
    const TokenPos tp = token_pos_wave(b, t);
    r = tp.r;
    n = tp.n;
  }
  int32_t* out = topk + (size_t)t * ldo;
  if (n <= k) {
    for (int j = threadIdx.x; j < k; j += NT) out[j] = j < n ? j : -1;
    return;
  }
  const int nsl = min((n + ks.cap - 1) / ks.cap, ks.nslots);
  for (int i = threadIdx.x; i < kBins1; i += NT) sm->hist[i] = 0u;   // counted during the gather
  if (threadIdx.x == 0) sm->misc[3] = 0u;
  // slot offsets, T = the largest threshold, the largest key
  if (nsl <= 64) {
    if (threadIdx.x < 64) {
      const int c = threadIdx.x;
      const uint32_t v = c < nsl ? min(v0, cap) : 0u;
      const uint32_t incl = wave_sum_incl(v);
      const uint32_t tv = wave_max(c < nsl ? tv0 : 0u), mx = wave_max(c < nsl ? mx0 : 0u);
      if (c < nsl) sm->pre[c] = incl - v;
      if (c == 63) { sm->pre[nsl] = incl; sm->misc[0] = tv; sm->misc[1] = mx; }
    }
  } else {
    if (threadIdx.x == 0) { sm->misc[0] = 0u; sm->misc[1] = 0u; }
    const int per = (nsl + NT - 1) / NT;
    const int a0 = min(nsl, per * (int)threadIdx.x), a1 = min(nsl, a0 + per);
    uint32_t sum = 0, tv = 0, mx = 0;
    for (int c = a0; c < a1; ++c) {
      sum += min(ks.counts[rbase + c], cap);
      tv = max(tv, ks.taus[rbase + c]);
      mx = max(mx, ks.maxes[rbase + c]);
    }
    uint32_t total;
    uint32_t run = block_scan_excl<NT>(sum, &total, sm->scratch);   // orders misc's reset first
    for (int c = a0; c < a1; ++c) { sm->pre[c] = run; run += min(ks.counts[rbase + c], cap); }
    if (threadIdx.x == 0) sm->pre[nsl] = total;
    atomicMax(&sm->misc[0], tv);
    atomicMax(&sm->misc[1], mx);
  }
  __syncthreads();
  const uint32_t C = sm->pre[nsl];
  const uint32_t T = sm->misc[0];
  const uint32_t kmax = sm->misc[1];
  auto at = [&](uint32_t i) {                   // workspace index of candidate i (position order)
    int lo = 0, hi = nsl - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm->pre[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return (rbase + lo) * cap + (i - sm->pre[lo]);
  };
  bool decided = false;                         // step 2 settled the row
  if (C <= (uint32_t)kResCap) {
    // The gather also counts the keys >= T in a histogram of up to 2048 bins
    // of (key - T) >> shift, which spans [T, kmax].
    const int width = kmax == T ? 0 : 32 - __clz(kmax - T);
    const int shift = width > 11 ? width - 11 : 0;
    auto put = [&](uint32_t i, uint2 e) {
      sm->ckey[i] = e.x;
      sm->cpos[i] = (int32_t)e.y;
      if (e.x >= T) atomicAdd(&sm->hist[(e.x - T) >> shift], 1u);
    };
    if (nsl <= nsp) {                           // every slot of the row was preloaded
      const uint32_t cnt = sm->pre[my_slot + 1] - sm->pre[my_slot], at0 = sm->pre[my_slot];
      if (my_ok && my_slot < nsl) {
#pragma unroll
        for (int u = 0; u < kSpecPer; ++u) {
          const uint32_t j = (uint32_t)(my_lane + tps * u);
          if (j < cnt) put(at0 + j, sc[u]);
        }
        const size_t sb = (rbase + my_slot) * cap;   // entries beyond the preloaded ones
        for (uint32_t j = (uint32_t)(my_lane + tps * kSpecPer); j < cnt; j += (uint32_t)tps)
          put(at0 + j, ks.cand[sb + j]);
      }
    } else {
      for (uint32_t i = threadIdx.x; i < C; i += NT) put(i, ks.cand[at(i)]);
    }
    __syncthreads();
    RowRun<NT> run;                             // this wave's run of the candidates
    run.load(sm->ckey, sm->cpos, C);
    // The bin of the k-th largest key: wave 0 finds it and passes it on (with
    // 16 waves per CU, every wave searching on its own costs more issue time
    // than the barrier).
    uint32_t above, in_bin, in_range;
    const uint32_t d = block_digit<NT>(sm->hist, 1 << (width - shift), (uint32_t)k, &above, &in_bin,
                                       &in_range, sm->scratch + NT / 64);
    if (in_range >= (uint32_t)k) {              // at least k candidates at or above T
      const uint32_t need = (uint32_t)k - above;
      const uint32_t base = T + (d << shift);
      uint32_t kstar, take;
      if (shift == 0) {                         // the bin is one key
        kstar = base;
        take = need;
      } else if (in_bin <= 64u) {               // rank the bin's keys: collected, then by wave 0
#pragma unroll
        for (int e = 0; e < RowRun<NT>::E; ++e) {
          if (e >= run.ne) break;
          const uint32_t x = run.key[e];
          if (run.valid(e) && x >= base && ((x - base) >> shift) == 0u) {
            const uint32_t j = atomicAdd(&sm->misc[3], 1u);
            if (j < 64u) sm->bucket[j] = x;
          }
        }
        __syncthreads();
        if (threadIdx.x < 64) {
          const int lane = threadIdx.x;
          const uint32_t x = (uint32_t)lane < in_bin ? sm->bucket[lane] : 0u;
          uint32_t gt = 0u, ge = 0u;
          for (int j = 0; j < (int)in_bin; ++j) {
            const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, j);
            gt += y > x;
            ge += y >= x;
          }
          const int L = __ffsll((unsigned long long)__ballot((uint32_t)lane < in_bin && gt < need &&
                                                             need <= ge)) - 1;
          if (lane == 0) {
            sm->misc[2] = (uint32_t)__builtin_amdgcn_readlane((int)x, L);
            sm->misc[3] = need - (uint32_t)__builtin_amdgcn_readlane((int)gt, L);
          }
        }
        __syncthreads();
        kstar = sm->misc[2];
        take = sm->misc[3];
      } else {                                  // a crowded bin: the general select within it
        __syncthreads();                        // every wave has read the histogram
        const uint32_t top = (uint32_t)min((uint64_t)kmax, (uint64_t)base + ((1ull << shift) - 1ull));
        kstar = select_kth_range<NT>(sm->ckey, C, need, base, top, &take, sm->hist, sm->bucket,
                                     sm->scratch);
      }
      emit_row_waves<NT>(run, kstar, take, k, out, sm->emit);
      decided = true;
    }
  } else {                                      // too many for LDS: select in place
    uint32_t above = 0u;
    for (uint32_t i = threadIdx.x; i < C; i += NT) above += ks.cand[at(i)].x >= T;
    above = wave_sum(above);
    if (threadIdx.x == 0) sm->misc[2] = 0u;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) atomicAdd(&sm->misc[2], above);
    __syncthreads();
    if (sm->misc[2] >= (uint32_t)k) {
      uint32_t take;
      const uint32_t kstar = radix_kth<NT, 3>([&](auto&& fn) {
        for (uint32_t i = threadIdx.x; i < C; i += NT) {
          const uint32_t key = ks.cand[at(i)].x;
          if (key >= T) fn(key);
        }
      }, (uint32_t)k, &take, sm->hist, sm->scratch);
      emit_ordered<NT>([&](uint32_t i) {
        const size_t a = at(i);
        return ks.cand[a];
      }, C, kstar, take, k, out, sm->scratch);
      decided = true;
    }
  }
  if (decided) return;
  // Step 3: the row's own slots (nslots * cap entries of 8 bytes, n <=
  // nslots * cap) take its rescored keys as one flat array of n words.
  __syncthreads();                              // the candidates' LDS is reused
  uint32_t* keys = reinterpret_cast<uint32_t*>(ks.cand + rbase * cap);
  rescore_row<FP4>(q8, w, cache, b, t, r, n, keys, reinterpret_cast<RescoreLds*>(smem));
  __syncthreads();                              // every key written before any is read
  uint32_t take;
  const uint32_t kstar = radix_kth<NT, 3>([&](auto&& fn) {
    for (int i = threadIdx.x; i < n; i += NT) fn(keys[i]);
  }, (uint32_t)k, &take, sm->hist, sm->scratch);
  emit_ordered<NT>([&](uint32_t i) { return make_uint2(keys[i], i); }, (uint32_t)n, kstar, take, k,
                   out, sm->scratch);
}

}  // namespace

// Blocks per chunk of the fused path: about one chunk per CU over the batch,
// 8 to kDynMaxBlocks blocks.
static int keep_chunk_blocks(const BatchArgs& b) {
  const int64_t blocks_per_row = (b.max_seq_len + kBlock - 1) / kBlock;
  const int64_t cb = (blocks_per_row * b.num_tokens + 255) / 256;
  return (int)std::min<int64_t>(kDynMaxBlocks, std::max<int64_t>(8, cb));
}

bool keep_path(const BatchArgs& b, int64_t dec_tokens) {
  const bool decode_split = b.max_query_len <= 1 || dec_tokens >= b.num_tokens;
  if (!decode_split || !topk_uses_long_rows(b.num_tokens, b.max_seq_len)) return false;
  const int cb = keep_chunk_blocks(b);
  const int64_t nslots = (b.max_seq_len + (int64_t)cb * kBlock - 1) / ((int64_t)cb * kBlock);
  return nslots <= kMaxSlots;
}

size_t keep_workspace_layout(const BatchArgs& b, void* base, KeepSlots* ks) {
  const int cb = keep_chunk_blocks(b);
  const int64_t cap = (int64_t)cb * kBlock;
  const int64_t nslots = std::max<int64_t>(1, (b.max_seq_len + cap - 1) / cap);
  const size_t T = (size_t)b.num_tokens;
  size_t off = 0;
  const size_t o_cand = off;
  off = align_up(off + sizeof(uint2) * T * nslots * cap, 256);
  const size_t o_cnt = off;
  off = align_up(off + sizeof(uint32_t) * T * nslots, 256);
  const size_t o_tau = off;
  off = align_up(off + sizeof(uint32_t) * T * nslots, 256);
  const size_t o_max = off;
  off = align_up(off + sizeof(uint32_t) * T * nslots, 256);
  if (base && ks) {
    char* p = static_cast<char*>(base);
    ks->cand = reinterpret_cast<uint2*>(p + o_cand);
    ks->counts = reinterpret_cast<uint32_t*>(p + o_cnt);
    ks->taus = reinterpret_cast<uint32_t*>(p + o_tau);
    ks->maxes = reinterpret_cast<uint32_t*>(p + o_max);
    ks->nslots = (int32_t)nslots;
    ks->cap = (int32_t)cap;
    ks->chunk_blocks = cb;
  }
  return off;
}

template <bool FP4>
hipError_t launch_keep_dyn(const dim3& grid, const uint8_t* q8, const float* w,
                           const CacheArgs& cache, const BatchArgs& b, int ident, const NewRows& nk,
                           bool fk, int k, const KeepSlots& ks, hipStream_t stream) {
  const bool big = ks.chunk_blocks > 64;
  const char* name = FP4 ? "score_keep_fp4_kernel" : "score_keep_kernel";   // the step's trace names
  if (fk && !big)
    IDX_LAUNCH(name, (score_keep_dyn_kernel<IDX_DYN_RING, true, 64, FP4>), grid,
               dim3(kDynThreads), stream, q8, w, cache, b, ks.chunk_blocks, ident, nk, k, ks);
  else if (fk)
    IDX_LAUNCH(name, (score_keep_dyn_kernel<IDX_DYN_RING, true, kDynMaxBlocks, FP4>),
               grid, dim3(kDynThreads), stream, q8, w, cache, b, ks.chunk_blocks, ident, nk, k, ks);
  else if (!big)
    IDX_LAUNCH(name, (score_keep_dyn_kernel<IDX_DYN_RING, false, 64, FP4>), grid,
               dim3(kDynThreads), stream, q8, w, cache, b, ks.chunk_blocks, ident, nk, k, ks);
  else
    IDX_LAUNCH(name, (score_keep_dyn_kernel<IDX_DYN_RING, false, kDynMaxBlocks, FP4>),
               grid, dim3(kDynThreads), stream, q8, w, cache, b, ks.chunk_blocks, ident, nk, k, ks);
  return hipGetLastError();
}

hipError_t launch_keep_candidates(const uint8_t* q8, const float* w, const CacheArgs& cache,
                                  const BatchArgs& b, const uint16_t* kq, int64_t kq_stride,
                                  const int64_t* slots, uint8_t* cache_w, int k,
                                  const KeepSlots& ks, hipStream_t stream, bool fp4) {
  if (b.num_tokens == 0) return hipSuccess;
  const int ident = b.num_reqs == b.num_tokens && b.max_query_len <= 1;
  if (b.max_seq_len > 0) {
    const dim3 grid((unsigned)ks.nslots, (unsigned)b.num_tokens);
    const NewRows nk = kq != nullptr ? NewRows{kq, kq_stride, slots, cache_w, cache.num_blocks * kBlock}
                                     : NewRows{};
    return fp4 ? launch_keep_dyn<true>(grid, q8, w, cache, b, ident, nk, kq != nullptr, k, ks, stream)
               : launch_keep_dyn<false>(grid, q8, w, cache, b, ident, nk, kq != nullptr, k, ks, stream);
  }
  if (kq != nullptr)
    return fp4 ? launch_quant_write_k_fp4(kq, b.num_tokens, kq_stride, slots, cache_w,
                                          cache.num_blocks * kBlock, stream)
               : launch_quant_write_k(kq, b.num_tokens, kq_stride, slots, cache_w,
                                      cache.num_blocks * kBlock, stream);
  return hipSuccess;
}

hipError_t launch_keep_select(const uint8_t* q8, const float* w, const CacheArgs& cache,
                              const BatchArgs& b, int k, const KeepSlots& ks, int32_t* out,
                              int64_t ldo, hipStream_t stream, bool fp4) {
  if (b.num_tokens == 0) return hipSuccess;
  const int ident = b.num_reqs == b.num_tokens && b.max_query_len <= 1;
  if (fp4)
    IDX_LAUNCH("topk_keep_resolve_kernel", (topk_keep_resolve_kernel<true>),
               dim3((unsigned)b.num_tokens), dim3(kResThreads), stream, q8, w, cache, b, ident, k, ks,
               out, ldo);
  else
    IDX_LAUNCH("topk_keep_resolve_kernel", (topk_keep_resolve_kernel<false>),
               dim3((unsigned)b.num_tokens), dim3(kResThreads), stream, q8, w, cache, b, ident, k, ks,
               out, ldo);
  return hipGetLastError();
}

}  // namespace idx

// Lightning-indexer scoring kernels (the method and its arithmetic are
// described in score_device.hpp) and their launchers.

#include "common.hpp"
#include "launch.hpp"
#include "score_device.hpp"

namespace idx {
namespace {

// ------------------------------------------------------------ prefill --
// A work-group takes kPrefillTM consecutive query tokens of one request
// (kPrefillTPW per wave) and `chunk_blocks` blocks of positions.  Each K block
// is fetched once per work-group: the work-group copies it with whole-line
// loads into one of two LDS slots (`lds`: 2 * kBlockBytes) and every wave reads
// its MFMA operands from there.  Tokens below `tok_lo` are left to the decode
// work split of a mixed launch.
__device__ __forceinline__ void prefill_body(int bx, int gy, int tok_lo,
                                             const uint8_t* __restrict__ q8,
                                             const float* __restrict__ w, const CacheArgs& cache,
                                             const BatchArgs& b, float* __restrict__ logits,
                                             int64_t ld, int chunk_blocks, int gpr,
                                             uint8_t* lds, float* __restrict__ samp) {
  constexpr int TPW = kPrefillTPW, NW = 4;
  PrefillGroup pg;
  if (!prefill_group(b, gy, tok_lo, gpr, &pg)) return;
  const int r = pg.r;
  const int q0 = pg.q0;
  const int nq = pg.nq;
  const int tb = pg.t0 - q0;                    // the group's tokens: tb .. tb + pg.nt - 1 of r
  const int L = pg.len;
  auto count = [&](int i) {
    int n = L - nq + i + 1;
    n = n < 0 ? 0 : n;
    return n > b.max_seq_len ? b.max_seq_len : n;
  };
  const int n_max = count(tb + pg.nt - 1);
  const int lb0 = bx * chunk_blocks;
  if (lb0 * kBlock >= n_max) return;
  const int nblk = min(chunk_blocks, (n_max - lb0 * kBlock + kBlock - 1) / kBlock);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
  const int lp = lane_pos(lane);
  uint8_t* kbuf0 = lds;
  uint8_t* kbuf1 = lds + kBlockBytes;
  // pbl[w] of lane i holds the physical block of the chunk's (64w + i)-th
  // block, read before the q loads so the first K loads wait on them alone
  int pbl[kPrefillWin];
#pragma unroll
  for (int w = 0; w < kPrefillWin; ++w)
    pbl[w] = 64 * w + lane < nblk ? (int)phys_block(b, cache, r, lb0 + 64 * w + lane) : -1;

  // Per token only wave-uniform integers are kept (the row pointers are formed
  // where they are used), so they live in scalar registers.
  QFrag f[TPW];
  int nt[TPW];
  int tk[TPW];                                  // batch index of the token (0 when absent)
  int sS[TPW], sSh[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int i = tb + wave * TPW + j;
    const int t = q0 + i;
    if (i < tb + pg.nt && t >= tok_lo && t < b.num_tokens) {
      load_q(f[j], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
      nt[j] = count(i);
      tk[j] = t;
    } else {
      zero_q(f[j]);
      nt[j] = 0;
      tk[j] = 0;
    }
    sS[j] = sample_stride(nt[j]);
    sSh[j] = 31 - __clz(sS[j]);
  }
  auto out = [&](int j) { return logits + (size_t)tk[j] * ld; };
  auto srow = [&](int j) { return samp + (size_t)tk[j] * kMaxSample; };   // compact sample copy

  if (cache.num_blocks == 0) {                  // no K at all: every score is 0
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj)
      for (int j = 0; j < nblk; ++j) {
        const int s = (lb0 + j) * kBlock + lp;
        if (s < nt[jj]) out(jj)[s] = 0.f;
        if (samp != nullptr) {
          const int sj = s >> sSh[jj];
          if (s < nt[jj] && (s & (sS[jj] - 1)) == ((37 * sj + 11) & (sS[jj] - 1))) srow(jj)[sj] = 0.f;
        }
      }
    return;
  }
  // block min(j, nblk-1) (past the last block it is re-read, from L2, so the
  // loop body issues its loads unconditionally)
  auto stage = [&](StageRegs<NW>& st, int j) {
    const int jc = min(j, nblk - 1);
    int v = pbl[0];
#pragma unroll
    for (int w = 1; w < kPrefillWin; ++w) v = (jc >> 6) == w ? pbl[w] : v;   // wave-uniform choice
    const int pb = __builtin_amdgcn_readlane(v, jc & 63);
    stage_load<NW>(st, cache.data + (int64_t)max(pb, 0) * kBlockBytes, pb >= 0);
  };

  // One set of staging registers: in iteration j it stores block j+1 into LDS
  // and takes block j+2's loads, which are in flight while block j is scored.
  StageRegs<NW> st;
  stage(st, 0);
  LinFrag lf;
  make_lin<TPW>(lf, f, lds + 2 * kBlockBytes + wave * kLinScratch, lane);
  stage_store<NW>(st, kbuf0);
  stage(st, 1);
  const int iters = (nblk + 1) & ~1;
  for (int j0 = 0; j0 < iters; j0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = j0 + u;
      __syncthreads();                     // block j in slot j&1; slot (j+1)&1 free
      stage_store<NW>(st, (j + 1) & 1 ? kbuf1 : kbuf0);   // unused past the end
      stage(st, j + 2);
      if (j >= nblk) continue;
      const uint8_t* kslot = j & 1 ? kbuf1 : kbuf0;
      const float ks = *reinterpret_cast<const float*>(kslot + kCodeBytes + lp * 4);
      float v[TPW];
      block_scores_with<TPW>(f, lf, [&](int tl) { return lds_tile(kslot, tl, lane); }, ks, v);
      const int s = (lb0 + j) * kBlock + lp;
#pragma unroll
      for (int jj = 0; jj < TPW; ++jj) {
        // non-temporal: the scores are read again only after the whole launch,
        // and streaming them out keeps L2 for the staged K blocks (~1.5%)
        if (s < nt[jj]) __builtin_nontemporal_store(v[jj], out(jj) + s);
        if (samp != nullptr) {
          const int sj = s >> sSh[jj];
          if (s < nt[jj] && (s & (sS[jj] - 1)) == ((37 * sj + 11) & (sS[jj] - 1))) srow(jj)[sj] = v[jj];
        }
      }
    }
  }
}

// The same work with each K block copied by the memory system straight into
// LDS (buffer loads to LDS): no staging registers, LDS stores or masking in
// the loop.  Three slots of 12 KiB (every wave issues three 1 KiB copies;
// lanes past the block's 528 chunks read past the buffer and write zeros into
// the slot's tail), so in iteration j block j is scored while blocks j+1 and
// j+2 are in flight: two blocks of compute hide the copies even when K comes
// from HBM (after the top-k has streamed the scores through the caches; with
// one block of look-ahead the step took 2.07 ms against 1.80).
// The copies are issued in inline assembly (m0 holds the LDS address), so the
// compiler, which does not see them, does not drain every memory operation at
// each barrier as it does for the builtin form.  The waits are placed by
// count instead: per iteration each wave issues exactly three copies and then
// exactly 2 * TPW stores (range-checked buffer stores, none behind a branch),
// and before block j is read each wave waits until only the operations it
// issued after block j's copies may be in flight (a wave's vector memory
// operations complete in issue order, which the compiler's own waits rely on
// too).  Copies of blocks past the chunk read nothing and fill unused slots.
constexpr int kDmaSlot = 12 * 1024;
constexpr int kPrefillDmaLds = 3 * kDmaSlot + 4 * kLinScratch;

// A buffer descriptor built from wave-uniform values, so that it sits in
// SGPRs (a descriptor the compiler cannot prove uniform gets a loop around
// every access that uses it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return byte_rsrc(reinterpret_cast<const void*>((uintptr_t)(((uint64_t)hi << 32) | lo)),
                   __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from rsrc + voff into LDS at m0 + 16 * lane (m0 is saved
// and restored around the copy; a write of m0 needs one wait state before an
// LDS copy reads it, as the compiler itself places).  The load has no VGPR
// result, so nothing of the wave's registers is written while it is in flight.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}

__device__ __forceinline__ void prefill_body_dma(int bx, int gy, const uint8_t* __restrict__ q8,
                                                 const float* __restrict__ w, const CacheArgs& cache,
                                                 const BatchArgs& b, float* __restrict__ logits,
                                                 int64_t ld, int chunk_blocks, int gpr,
                                                 uint8_t* lds, float* __restrict__ samp) {
  constexpr int TPW = kPrefillTPW, NW = 4;
  PrefillGroup pg;
  if (!prefill_group(b, gy, 0, gpr, &pg)) return;
  const int r = pg.r;
  const int q0 = pg.q0;
  const int nq = pg.nq;
  const int tb = pg.t0 - q0;
  const int L = pg.len;
  auto count = [&](int i) {
    int n = L - nq + i + 1;
    n = n < 0 ? 0 : n;
    return n > b.max_seq_len ? b.max_seq_len : n;
  };
  const int n_max = count(tb + pg.nt - 1);
  const int lb0 = bx * chunk_blocks;
  if (lb0 * kBlock >= n_max) return;
  const int nblk = min(chunk_blocks, (n_max - lb0 * kBlock + kBlock - 1) / kBlock);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lp = lane_pos(lane);
  int pbl[kPrefillWin];
#pragma unroll
  for (int w = 0; w < kPrefillWin; ++w)
    pbl[w] = 64 * w + lane < nblk ? (int)phys_block(b, cache, r, lb0 + 64 * w + lane) : -1;

  QFrag f[TPW];
  int nt[TPW];
  int tk[TPW];
  int sS[TPW], sSh[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int i = tb + wave * TPW + j;
    const int t = q0 + i;
    if (i < tb + pg.nt && t < b.num_tokens) {
      load_q(f[j], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
      nt[j] = count(i);
      tk[j] = t;
    } else {
      zero_q(f[j]);
      nt[j] = 0;
      tk[j] = 0;
    }
    sS[j] = sample_stride(nt[j]);
    sSh[j] = 31 - __clz(sS[j]);
  }
  if (cache.num_blocks == 0) {                  // no K at all: every score is 0
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj)
      for (int j = 0; j < nblk; ++j) {
        const int s = (lb0 + j) * kBlock + lp;
        float* o = logits + (size_t)tk[jj] * ld;
        if (s < nt[jj]) o[s] = 0.f;
        if (samp != nullptr) {
          const int sj = s >> sSh[jj];
          if (s < nt[jj] && (s & (sS[jj] - 1)) == ((37 * sj + 11) & (sS[jj] - 1)))
            samp[(size_t)tk[jj] * kMaxSample + sj] = 0.f;
        }
      }
    return;
  }
  // the token rows and their sample copies as range-checked buffers: a
  // position past the token's causal range, or not sampled, is stored past
  // the buffer's end and dropped
  __amdgpu_buffer_rsrc_t orow[TPW], srs[TPW];
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    orow[jj] = uniform_rsrc(logits + (size_t)tk[jj] * ld, nt[jj] * 4);
    srs[jj] = uniform_rsrc(samp != nullptr ? samp + (size_t)tk[jj] * kMaxSample : logits,
                           samp != nullptr && nt[jj] > 0 ? kMaxSample * 4 : 0);
  }
  LinFrag lf;
  make_lin<TPW>(lf, f, lds + 3 * kDmaSlot + wave * kLinScratch, lane);

  // block j of the chunk into `slot` (from nblk on, or absent: zeros)
  auto copy_block = [&](int j, uint8_t* slot) {
    const int jc = min(j, nblk - 1);
    int v = pbl[0];
#pragma unroll
    for (int w = 1; w < kPrefillWin; ++w) v = (jc >> 6) == w ? pbl[w] : v;
    const int pb = __builtin_amdgcn_readlane(v, jc & 63);
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(cache.data + (int64_t)max(pb, 0) * kBlockBytes,
                                                   (j < nblk && pb >= 0) ? kBlockBytes : 0);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int u = wave + NW * i;
      const int ci = 64 * u + lane;
      const uint32_t voff = ci < kBlockBytes / 16 ? (uint32_t)stage_src<NW>(ci) : (uint32_t)kPastBlock;
      copy_to_lds(rs, voff, __builtin_amdgcn_readfirstlane(lds_address(slot + u * 1024)));
    }
  };
  uint8_t* slot0 = lds;
  uint8_t* slot1 = lds + kDmaSlot;
  uint8_t* slot2 = lds + 2 * kDmaSlot;
  copy_block(0, slot0);
  copy_block(1, slot1);
  static_assert(TPW == 2, "the waits below count 2 * TPW stores per iteration");
  for (int j = 0; j < nblk; ++j) {
    // operations after block j's copies: block j+1's copies and the stores
    // of the iterations in between
    if (j == 0) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (j == 1) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");    // 3 + 2 * TPW
    else asm volatile("s_waitcnt vmcnt(11)" ::: "memory");               // 3 + 4 * TPW
    __syncthreads();                            // block j in slot0; slot2 read last in j-1
    copy_block(j + 2, slot2);
    const uint8_t* cur = slot0;
    const float ks = *reinterpret_cast<const float*>(cur + kCodeBytes + lp * 4);
    float v[TPW];
    block_scores_with<TPW>(f, lf, [&](int tl) { return lds_tile(cur, tl, lane); }, ks, v);
    const int s = (lb0 + j) * kBlock + lp;
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[jj]), orow[jj], (uint32_t)s * 4u, 0,
                                            kLoadStream);
      const int sj = s >> sSh[jj];
      const bool sampled = (s & (sS[jj] - 1)) == ((37 * sj + 11) & (sS[jj] - 1));
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[jj]), srs[jj],
                                            sampled && s < nt[jj] ? (uint32_t)sj * 4u : (uint32_t)kPastBlock * 16u,
                                            0, 0);
    }
    uint8_t* const t0 = slot0;
    slot0 = slot1;
    slot1 = slot2;
    slot2 = t0;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy lands after the work-group ends
}

// ------------------------------------------------------------ kernels --
template <int NB>
__global__ __launch_bounds__(kScoreThreads)
__attribute__((amdgpu_waves_per_eu(IDX_DECODE_WAVES_PER_EU))) void score_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    float* __restrict__ logits, int64_t ld, int chunk_blocks, int ident, float* samp) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kScoreLds];
  int cx, ry;
  xcd_spread(&cx, &ry);
  decode_body<NB, false>(cx, ry, q8, w, cache, b, logits, ld, chunk_blocks,
                         ident != 0, lds, NewRows{}, samp);
}

// Decode scoring of an F layer that also writes this step's new K rows.
template <int NB>
__global__ __launch_bounds__(kScoreThreads)
__attribute__((amdgpu_waves_per_eu(IDX_DECODE_WAVES_PER_EU))) void score_decode_write_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    float* __restrict__ logits, int64_t ld, int chunk_blocks, int ident, NewRows nk, float* samp) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kScoreLds];
  int cx, ry;
  xcd_spread(&cx, &ry);
  decode_body<NB, true>(cx, ry, q8, w, cache, b, logits, ld, chunk_blocks,
                        ident != 0, lds, nk, samp);
}

// two work-groups per CU: the register budget is 256 VGPRs
#ifndef IDX_PREFILL_DMA
#define IDX_PREFILL_DMA 1
#endif
__global__ __launch_bounds__(kScoreThreads)
__attribute__((amdgpu_waves_per_eu(2))) void score_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    float* __restrict__ logits, int64_t ld, int chunk_blocks, int gpr, float* samp) {
  int cx, ry;
  xcd_spread(&cx, &ry);
  if constexpr (IDX_PREFILL_DMA) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kPrefillDmaLds];
    prefill_body_dma(cx, ry, q8, w, cache, b, logits, ld, chunk_blocks, gpr, lds, samp);
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kPrefillLds];
    prefill_body(cx, ry, 0, q8, w, cache, b, logits, ld, chunk_blocks, gpr, lds, samp);
  }
}

// Mixed batch in one launch: rows y < dec_tokens are tokens scored with the
// decode split, the rest are prefill groups; the two kinds of work-group share
// the machine (HBM-bound decode beside MFMA-bound prefill).
template <int NB>
__global__ __launch_bounds__(kScoreThreads)
__attribute__((amdgpu_waves_per_eu(2))) void score_mixed_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    float* __restrict__ logits, int64_t ld, int dec_tokens, int dec_chunk_blocks,
    int pre_chunk_blocks, int gpr, float* samp) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kScoreLds];
  int cx, ry;
  xcd_spread(&cx, &ry);
  if (ry < dec_tokens)
    decode_body<NB, false, true>(cx, ry, q8, w, cache, b, logits, ld, dec_chunk_blocks,
                                 false, lds, NewRows{}, samp);
  else
    prefill_body(cx, ry - dec_tokens, dec_tokens, q8, w, cache, b, logits, ld,
                 pre_chunk_blocks, gpr, lds, samp);
}

}  // namespace

#ifndef IDX_DECODE_WG_PER_CU
#define IDX_DECODE_WG_PER_CU 2
#endif
constexpr int64_t kDecodeSlots = 256 * IDX_DECODE_WG_PER_CU;   // resident decode work-groups

// Decode chunk: about two work-groups per CU over the decode tokens (two fit
// by registers), at least 8 and at most 64 blocks per work-group.
int decode_chunk_blocks(int max_seq_len, int64_t tokens) {
  const int64_t blocks_per_row = (max_seq_len + kBlock - 1) / kBlock;
  const int64_t total = blocks_per_row * tokens;
  int64_t cb = (total + kDecodeSlots - 1) / kDecodeSlots;
  cb = (cb + 3) / 4 * 4;
  return (int)std::min<int64_t>(64, std::max<int64_t>(8, cb));
}

bool score_writes_k(const BatchArgs& b, int64_t dec_tokens) {
  return b.max_query_len <= kMaxFusedRows && (b.max_query_len <= 1 || dec_tokens >= b.num_tokens);
}

hipError_t launch_score_write_k(const uint8_t* q8, const float* w, const CacheArgs& cache,
                                const BatchArgs& b, const uint16_t* k, int64_t k_stride,
                                const int64_t* slots, uint8_t* cache_w, float* logits, int64_t ld,
                                float* samp, hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  if (b.max_seq_len == 0) return launch_quant_write_k(k, b.num_tokens, k_stride, slots, cache_w,
                                                      cache.num_blocks * kBlock, stream);
  const int cb = decode_chunk_blocks(b.max_seq_len, b.num_tokens);
  const int chunks = (b.max_seq_len + cb * kBlock - 1) / (cb * kBlock);
  const dim3 grid((unsigned)chunks, (unsigned)b.num_tokens);
  const NewRows nk{k, k_stride, slots, cache_w, cache.num_blocks * kBlock};
  const int ident = b.num_reqs == b.num_tokens && b.max_query_len <= 1;
  IDX_LAUNCH("score_decode_write_kernel", (score_decode_write_kernel<IDX_DECODE_RING>), grid,
             dim3(kScoreThreads), stream, q8, w, cache, b, logits, ld, cb, ident, nk, samp);
  return hipGetLastError();
}

hipError_t launch_score(const uint8_t* q8, const float* w, const CacheArgs& cache,
                        const BatchArgs& b, int64_t dec_tokens, float* logits, int64_t ld,
                        float* samp, hipStream_t stream) {
  if (b.num_tokens == 0 || b.max_seq_len == 0) return hipSuccess;
  if (b.max_query_len <= 1) dec_tokens = b.num_tokens;
  if (dec_tokens >= b.num_tokens) {
    const int cb = decode_chunk_blocks(b.max_seq_len, b.num_tokens);
    const int chunks = (b.max_seq_len + cb * kBlock - 1) / (cb * kBlock);
    const dim3 grid((unsigned)chunks, (unsigned)b.num_tokens);
    IDX_LAUNCH("score_decode_kernel", (score_decode_kernel<IDX_DECODE_RING>), grid,
               dim3(kScoreThreads), stream, q8, w, cache, b, logits, ld, cb,
               (int)(b.num_reqs == b.num_tokens && b.max_query_len <= 1), samp);
  } else {
    if (dec_tokens < 0) dec_tokens = 0;
    // groups numbered per request (gpr each) when that wastes little, else
    // numbered across the batch (a scan finds each group's request)
    const int64_t per_req = (int64_t)((b.max_query_len + kPrefillTM - 1) / kPrefillTM);
    const int64_t flat = prefill_groups_bound(b.num_tokens - dec_tokens, b.num_reqs);
    const bool arith = per_req * b.num_reqs <= flat + flat / 4;
    const int gpr = arith ? (int)per_req : 0;
    const int64_t groups = arith ? per_req * b.num_reqs : flat;
    if (dec_tokens + groups > 65535) return hipErrorInvalidConfiguration;   // grid y-extent
    const int dcb = decode_chunk_blocks(b.max_seq_len, dec_tokens);
    const int dchunks = (b.max_seq_len + dcb * kBlock - 1) / (dcb * kBlock);
    const int pcb = prefill_chunk_blocks(b, groups, dec_tokens * dchunks >= kDecodeSlots);
    const int pchunks = (b.max_seq_len + pcb * kBlock - 1) / (pcb * kBlock);
    if (dec_tokens == 0) {
      const dim3 grid((unsigned)pchunks, (unsigned)groups);
      IDX_LAUNCH("score_prefill_kernel", (score_prefill_kernel), grid, dim3(kScoreThreads),
                 stream, q8, w, cache, b, logits, ld, pcb, gpr, samp);
    } else {
      const dim3 grid((unsigned)std::max(dchunks, pchunks), (unsigned)(dec_tokens + groups));
      IDX_LAUNCH("score_mixed_kernel", (score_mixed_kernel<IDX_DECODE_RING>), grid,
                 dim3(kScoreThreads), stream, q8, w, cache, b, logits, ld, (int)dec_tokens, dcb,
                 pcb, gpr, samp);
    }
  }
  return hipGetLastError();
}

}  // namespace idx

// Device code of the FP4 indexer K cache (internal), shared by its
// quantise-and-scatter and scoring kernels (fp4.hip) and the fused score +
// top-k kernels (fused.hip).  The format and the scoring method are
// described in fp4.hip.
#pragma once

#include "common.hpp"
#include "quant_device.hpp"
#include "score_device.hpp"

namespace idx {
namespace {

constexpr int kFp4CodeBytes = kBlock * kHeadDim / 2;          // 4096
constexpr int kFp4BlockBytes = kFp4CodeBytes + kBlock * 4;     // 4352
constexpr int kFp4Plane = kBlock * 16;                          // one group's codes: 1024

// ---------------------------------------------------------- quantiser --

// Group exponent: the smallest e with max(amax, 1e-4) <= 6 * 2^e.  `amag` is
// the bf16 magnitude pattern of the group's amax: amax = (1 + m/128) 2^(E-127)
// and 6 = 1.5 * 2^2.
__device__ __forceinline__ int fp4_exponent(uint32_t amag) {
  const float a = __uint_as_float(amag << 16);
  if (!(a >= 1e-4f)) return -15;                 // the floor: 1e-4 <= 6 * 2^-15
  const int E = (int)(amag >> 7);
  const int m = (int)(amag & 0x7F);
  return (E - 127) - 2 + (m > 64 ? 1 : 0);
}

// E2M1 code of bf16 value x times s = 2^-e (exact in fp32; |x s| <= 6): the
// number of rounding boundaries at or below |x s|, each boundary open or
// closed so that a tie goes to the even code, plus the sign bit.
__device__ __forceinline__ uint32_t encode_e2m1(uint32_t x, float s) {
  const float y = fabsf(__uint_as_float(x << 16) * s);
  const uint32_t c = (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
                     (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
                     (uint32_t)(y > 5.f);
  return c | ((x >> 12) & 8u);
}

// ------------------------------------------------------------ scoring --

// One block's B operands for this lane: tile tl's 16 code bytes (position
// 16 tl + lane%16, group lane/16) and the dword of that position's group
// scales for the four tiles (byte tl).
struct KBlock4 {
  uint4 b[4];
  uint32_t sc;
};

// A buffer resource of `bytes` = 0 (absent block, or past the run) loads
// zeros: codes 0 score 0.
template <int AUX>
__device__ __forceinline__ void fp4_block_load(KBlock4& kb, const uint8_t* base, int bytes, int lane) {
  const __amdgpu_buffer_rsrc_t rs = byte_rsrc(base, bytes);
  const int c = lane & 15, G = lane >> 4;
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, G * kFp4Plane + (16 * tl + c) * 16, 0, AUX);
    kb.b[tl] = make_uint4(x[0], x[1], x[2], x[3]);
  }
  kb.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, kFp4CodeBytes + G * 64 + c * 4, 0, AUX);
}

template <int TL>
__device__ __forceinline__ v4f mfma_fp4(const v8i& a, const uint4& b, uint32_t sc) {
  const v8i bb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // A: E4M3 (format 0), scale 2^0; B: E2M1 (format 4), scale byte TL of sc
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, zero, 0, 4, 0, 127, TL, (int)sc);
}

// Tile TL of a block for NT tokens: this lane's partial (its 16 heads, its
// share of the linear half) into part[t][TL], in the FP8 path's order.
template <int TL, int NT>
__device__ __forceinline__ void fp4_tile(const QFrag* f, const LinFrag& lf, const KBlock4& kb,
                                         float (&part)[NT][4]) {
  const v4f lin = mfma_fp4<TL>(lf.a, kb.b[TL], kb.sc);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    TileAcc acc;
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) acc.d[hg] = mfma_fp4<TL>(f[t].a[hg], kb.b[TL], kb.sc);
    part[t][TL] = fmaf(lin[t], lf.sc[t], tile_epilogue(f[t], acc));
  }
}

// Scores of one block for NT tokens: out[t] is token t's score at position
// lane_pos(lane).
template <int NT>
__device__ __forceinline__ void fp4_block_scores(const QFrag* f, const LinFrag& lf, const KBlock4& kb,
                                                 float* out) {
  float part[NT][4];
  fp4_tile<0, NT>(f, lf, kb, part);
  fp4_tile<1, NT>(f, lf, kb, part);
  fp4_tile<2, NT>(f, lf, kb, part);
  fp4_tile<3, NT>(f, lf, kb, part);
#pragma unroll
  for (int t = 0; t < NT; ++t) out[t] = reduce_block(part[t][0], part[t][1], part[t][2], part[t][3]);
}

// Stores a score at position s of a row of n (and its sampled copy).
__device__ __forceinline__ void fp4_emit(float* __restrict__ out, float* __restrict__ srow, int s,
                                         int n, int sS, int sSh, float v) {
  if (s < n) out[s] = v;
  if (srow != nullptr) {
    const int sj = s >> sSh;
    if (s < n && (s & (sS - 1)) == ((37 * sj + 11) & (sS - 1))) srow[sj] = v;
  }
}

// A new K row quantised as the cache stores it, for this lane's group
// G = lane / 16 (dims 32G .. 32G+31 at kr): its 32 E2M1 codes, low nibble
// first, and the group's exponent e (scale byte e + 127).
__device__ __forceinline__ uint4 fp4_quant_group(const uint16_t* __restrict__ kr, int* e_out) {
  uint32_t x[16];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint2 p2 = *reinterpret_cast<const uint2*>(kr + 4 * v);
    x[2 * v] = p2.x;
    x[2 * v + 1] = p2.y;
  }
  uint32_t am = 0u;
#pragma unroll
  for (int v = 0; v < 16; ++v) am = max(am, max(x[v] & 0x7FFFu, (x[v] >> 16) & 0x7FFFu));
  const int e = fp4_exponent(am);
  const float sc = pow2f(-e);
  uint32_t c[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    c[d] = 0u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t wv = x[4 * d + m];
      c[d] |= encode_e2m1(wv & 0xFFFFu, sc) << (8 * m);
      c[d] |= encode_e2m1(wv >> 16, sc) << (8 * m + 4);
    }
  }
  *e_out = e;
  return make_uint4(c[0], c[1], c[2], c[3]);
}

// Row `slot` of the FP4 cache from each group's codes and exponent (lane
// 16G writes group G).
__device__ __forceinline__ void fp4_write_row(uint8_t* cache, int64_t slot, uint4 code, int e,
                                              int lane) {
  uint8_t* cb = cache + (slot / kBlock) * kFp4BlockBytes;
  const int p = (int)(slot % kBlock), G = lane >> 4;
  if ((lane & 15) == 0) {
    *reinterpret_cast<uint4*>(cb + G * kFp4Plane + p * 16) = code;
    cb[kFp4CodeBytes + G * 64 + (p & 15) * 4 + (p >> 4)] = (uint8_t)(e + 127);
  }
}

// The staged block's row r (lane (r % 16) of each group holds it) replaced by
// a new row's codes and exponent byte.
__device__ __forceinline__ void fp4_patch_row(KBlock4& kb, int r, uint4 code, uint32_t ebyte,
                                              int lane) {
  const int tl = r >> 4;
  const bool mine = (lane & 15) == (r & 15);
  // element-wise selects: an index into kb.b would put the block in scratch
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool put = mine && q == tl;
    kb.b[q].x = put ? code.x : kb.b[q].x;
    kb.b[q].y = put ? code.y : kb.b[q].y;
    kb.b[q].z = put ? code.z : kb.b[q].z;
    kb.b[q].w = put ? code.w : kb.b[q].w;
  }
  const uint32_t mask = 0xFFu << (8 * tl);
  kb.sc = mine ? (kb.sc & ~mask) | (ebyte << (8 * tl)) : kb.sc;
}

// Decode split: one query token per work-group, `chunk_blocks` blocks of its
// causal range split into four runs, one per wave.  The K stream is read
// once: each wave keeps NB-1 blocks' operand loads in flight, straight into
// the MFMA registers (non-temporal).  `ident`: token t is request t.
// Returns the token's causal count, or -1 when the chunk holds none of its
// positions.
template <int NB>
__device__ __forceinline__ int fp4_decode_body(int bx, int t, const uint8_t* __restrict__ q8,
                                               const float* __restrict__ w, const CacheArgs& cache,
                                               const BatchArgs& b, float* __restrict__ logits,
                                               int64_t ld, int chunk_blocks, bool ident,
                                               uint8_t* lds, float* __restrict__ samp) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  TokenPos tp;
  if (ident) {
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
  const int lb0 = bx * chunk_blocks;
  if (lb0 * kBlock >= n) return -1;
  const int nblk = min(chunk_blocks, (n - lb0 * kBlock + kBlock - 1) / kBlock);
  const int per = (nblk + 3) / 4;
  const int mine = max(0, min(per, nblk - wave * per));        // <= 16 blocks
  if (mine == 0) return n;
  auto blk = [&](int j) { return lb0 + wave * per + j; };
  const int pbl = lane < mine ? (int)phys_block(b, cache, tp.r, blk(lane)) : -1;
  auto load = [&](KBlock4& kb, int j) {                       // j <= mine + NB - 2 < 64
    const int pb = __builtin_amdgcn_readlane(pbl, j);
    fp4_block_load<kLoadStream>(kb, cache.data + (int64_t)max(pb, 0) * kFp4BlockBytes,
                                (j < mine && pb >= 0) ? kFp4BlockBytes : 0, lane);
  };
  KBlock4 ring[NB];
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) load(ring[u], u);
  LinFrag lf;
  make_lin<1>(lf, f, lds + wave * kLinScratch, lane);

  float* out = logits + (size_t)t * ld;
  float* srow = samp ? samp + (size_t)t * kMaxSample : nullptr;
  const int sS = sample_stride(n), sSh = 31 - __clz(sS);
  const int lp = lane_pos(lane);
  const int iters = (mine + NB - 1) / NB * NB;
  for (int j0 = 0; j0 < iters; j0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u;
      load(ring[(u + NB - 1) % NB], j + NB - 1);
      __builtin_amdgcn_sched_barrier(0);
      KBlock4& kb = ring[u];
      float v;
      fp4_block_scores<1>(f, lf, kb, &v);
      const int s = blk(j) * kBlock + lp;
      if (j < mine) fp4_emit(out, srow, s, n, sS, sSh, v);
    }
  }
  return n;
}

}  // namespace
}  // namespace idx

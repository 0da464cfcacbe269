// Device code of the lightning-indexer scoring kernels (internal), shared by
// the scoring kernels (score.hip) and the fused score + top-k kernels
// (fused.hip).
//
// Lightning-indexer scores on gfx950 matrix cores.
//
//   I[t, s] = ks[s] * sum_h w[t, h] * max(0, q8[t, h, :] . k8[s, :])
//
// (IndexCache blog post: SparseAttnIndexer / Indexer.forward -- 64 fp8 query
// heads share one fp8 K per position, folded fp32 weights; the score's form is
// the DSA lightning indexer's.)
//
// Work unit: one token x one 64-position K block (four 16-position tiles).
//  * Per tile, four v_mfma_f32_16x16x128_f8f6f4 (16 heads x 16 positions x 128
//    dims each).  Lane `lane` receives D[head 4*(lane/16)+i][position lane%16]
//    in register i.  Both operands use the same byte->k assignment (lane group
//    G = lane/16 holds k in [16G, 16G+16) and [64+16G, 64+16G+16)), so the
//    contraction covers all 128 dims whatever the hardware's k order is.
//  * The ReLU is split: w * max(d, 0) = (w/2) |d| + (w/2) d.  The first half
//    is one fma per MFMA output (the absolute value is a free source
//    modifier); each lane sums its 16 heads of a tile.  The second half, summed
//    over the heads, is linear in k: sum_h (w_h/2) q8[h] . k8 = u . k8 with
//    u = sum_h (w_h/2) q8[h] (fp32, once per token).  u is held as four E4M3
//    pieces, u ~= sum_j 2^(c-4j) p_j (each piece codes the previous residual,
//    so four of them carry about 16 significant bits), and one more MFMA per
//    tile contracts them with the same K operand for all of a wave's tokens.
//    Two accumulator sets alternate so the next tile's MFMAs run while the
//    previous tile's epilogue executes.
//  * The four per-tile partials (each split over the four lane groups) are
//    reduced and transposed at once with v_permlane32_swap / v_permlane16_swap:
//    afterwards lane `lane` holds the full 64-head sum of one position,
//    16*tile(lane/16) + lane%16 with tile(r) = {0, 2, 1, 3}[r].
//
// Every kernel computes a score with exactly this sequence of operations, so
// all kernels and entry points give bit-identical scores.  The matrix cores
// do not accumulate their 128 fp8 products exactly (about 2e-4 of
// sum |a_k b_k| at worst on gfx950); that, not the split's fp32 arithmetic,
// sets the scores' error.

#pragma once

#include "common.hpp"
#include "quant_device.hpp"

namespace idx {
namespace {


// One token's q as four A operands (16 heads each) plus this lane's 16 halved
// weights w[16*hg + 4*(lane/16) + i] / 2 in w[4*hg + i], and the halved weights
// of the heads whose q rows it holds, w[16*hg + lane%16] / 2 in wc[hg].
struct QFrag {
  v8i a[4];
  float w[16];
  float wc[4];
};

// The linear half's MFMA operand for up to four tokens of a wave: row 4j+t
// (lane%16) holds piece j of token t over this lane group's k range, and
// sc[t] = 2^(c_t - 4*(lane/16)) scales the output row this lane receives for
// token t (piece lane/16 of it).
struct LinFrag {
  v8i a;
  float sc[4];
};

// One 64-position block: the four tiles' B operands and the scale of the
// position this lane ends up holding.
struct KBlock {
  v8i b[4];
  float ks;
};

struct TileAcc {
  v4f d[4];
};

__device__ __forceinline__ int lane_pos(int lane) {
  const int r = lane >> 4;
  return 16 * (((r & 1) << 1) | (r >> 1)) + (lane & 15);
}

__device__ __forceinline__ v8i pack8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ void load_q(QFrag& f, const uint8_t* __restrict__ qt,
                                       const float* __restrict__ wt, int lane) {
  const int c = lane & 15, G = lane >> 4;
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    const uint8_t* row = qt + (hg * 16 + c) * kHeadDim;
    f.a[hg] = pack8(*reinterpret_cast<const uint4*>(row + 16 * G),
                    *reinterpret_cast<const uint4*>(row + 64 + 16 * G));
    const float4 wv = *reinterpret_cast<const float4*>(wt + hg * 16 + 4 * G);
    f.w[hg * 4 + 0] = 0.5f * wv.x; f.w[hg * 4 + 1] = 0.5f * wv.y;
    f.w[hg * 4 + 2] = 0.5f * wv.z; f.w[hg * 4 + 3] = 0.5f * wv.w;
    f.wc[hg] = 0.5f * wt[hg * 16 + c];
  }
}

__device__ __forceinline__ void zero_q(QFrag& f) {
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    f.a[hg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    f.wc[hg] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.w[hg * 4 + i] = 0.f;
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Builds the linear half's pieces for NT tokens (f[0..NT-1]); `scratch` is 4 KB
// of LDS owned by this wave.  Per token: each lane sums its four heads' halved
// weights times q over its lane group's 32 k values; the 16 lanes of a group
// (16 different heads each) are summed, quads by DPP and the four quads through
// LDS, so that each lane ends with u at two k values.  The exponent c is the
// smallest with max|u| <= 448 * 2^c (clamped to [-100, 100]); piece j codes the
// residual times 2^-(c-4j) to the nearest E4M3 value and the residual loses it.
// Every step runs in a fixed order, so a token's pieces do not depend on the
// other tokens of the wave or on which kernel builds them.  The tokens go
// through each step together, so their LDS round trips overlap.
template <int NT>
__device__ __forceinline__ void make_lin(LinFrag& lf, const QFrag* f, uint8_t* scratch, int lane) {
  static_assert(NT <= 2, "4 KB of scratch holds two tokens' partial sums");
  const int c = lane & 15, G = lane >> 4;
  float u0[NT], u1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float* part = reinterpret_cast<float*>(scratch) + t * 512;   // [G][quad][32] fp32: 2 KB
    float p[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) p[k] = 0.f;
#pragma unroll
    for (int hg = 0; hg < 4; ++hg)
#pragma unroll
      for (int dw = 0; dw < 8; ++dw) {
        const int x = f[t].a[hg][dw];
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
        p[4 * dw + 0] = fmaf(f[t].wc[hg], lo[0], p[4 * dw + 0]);
        p[4 * dw + 1] = fmaf(f[t].wc[hg], lo[1], p[4 * dw + 1]);
        p[4 * dw + 2] = fmaf(f[t].wc[hg], hi[0], p[4 * dw + 2]);
        p[4 * dw + 3] = fmaf(f[t].wc[hg], hi[1], p[4 * dw + 3]);
      }
    // quad sums (lane ^ 1, then lane ^ 2): additions commute exactly, so the
    // four lanes of a quad hold the same bits
#pragma unroll
    for (int k = 0; k < 32; ++k)
      p[k] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(p[k]), 0xB1, 0xF, 0xF, false));
#pragma unroll
    for (int k = 0; k < 32; ++k)
      p[k] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(p[k]), 0x4E, 0xF, 0xF, false));
    if ((c & 3) == 0) {                                       // one lane per quad stores its sums
      float4* dst = reinterpret_cast<float4*>(part + (G * 4 + (c >> 2)) * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[q] = make_float4(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
    }
  }
  wave_sync_lds();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float* part = reinterpret_cast<const float*>(scratch) + t * 512;
    const float2 a0 = *reinterpret_cast<const float2*>(part + (G * 4 + 0) * 32 + 2 * c);
    const float2 a1 = *reinterpret_cast<const float2*>(part + (G * 4 + 1) * 32 + 2 * c);
    const float2 a2 = *reinterpret_cast<const float2*>(part + (G * 4 + 2) * 32 + 2 * c);
    const float2 a3 = *reinterpret_cast<const float2*>(part + (G * 4 + 3) * 32 + 2 * c);
    u0[t] = ((a0.x + a1.x) + a2.x) + a3.x;
    u1[t] = ((a0.y + a1.y) + a2.y) + a3.y;
  }
  wave_sync_lds();                                            // the partial sums' space takes the codes
  uint8_t* pcs = scratch;                                     // [t][j][G][32] codes
  int ct[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // max |u| over the 128 k values: rotations within each row of 16 lanes,
    // then the four rows (max is exact in any order)
    int mb = (int)max(__float_as_uint(fabsf(u0[t])), __float_as_uint(fabsf(u1[t])));
    mb = max((uint32_t)mb, (uint32_t)__builtin_amdgcn_update_dpp(0, mb, 0x128, 0xF, 0xF, false));
    mb = max((uint32_t)mb, (uint32_t)__builtin_amdgcn_update_dpp(0, mb, 0x124, 0xF, 0xF, false));
    mb = max((uint32_t)mb, (uint32_t)__builtin_amdgcn_update_dpp(0, mb, 0x122, 0xF, 0xF, false));
    mb = max((uint32_t)mb, (uint32_t)__builtin_amdgcn_update_dpp(0, mb, 0x121, 0xF, 0xF, false));
    const uint32_t m = max(max((uint32_t)__builtin_amdgcn_readlane(mb, 0), (uint32_t)__builtin_amdgcn_readlane(mb, 16)),
                           max((uint32_t)__builtin_amdgcn_readlane(mb, 32), (uint32_t)__builtin_amdgcn_readlane(mb, 48)));
    int c0 = (int)((m >> 23) & 0xFF) - 127 - 8 + ((m & 0x7FFFFF) > 0x600000 ? 1 : 0);
    c0 = min(100, max(-100, c0));
    float r0 = u0[t], r1 = u1[t];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cj = c0 - 4 * j;
      const float down = __uint_as_float((uint32_t)(127 - cj) << 23);
      const float up = __uint_as_float((uint32_t)(127 + cj) << 23);
      const int code = __builtin_amdgcn_cvt_pk_fp8_f32(r0 * down, r1 * down, 0, false);
      const auto back = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
      r0 = fmaf(-back[0], up, r0);
      r1 = fmaf(-back[1], up, r1);
      *reinterpret_cast<uint16_t*>(pcs + ((t * 4 + j) * 4 + G) * 32 + 2 * c) = (uint16_t)code;
    }
    ct[t] = c0;
  }
  wave_sync_lds();
  {
    const int t = c & 3, j = c >> 2;
    if (t < NT) {
      const uint8_t* src = pcs + ((t * 4 + j) * 4 + G) * 32;
      lf.a = pack8(*reinterpret_cast<const uint4*>(src), *reinterpret_cast<const uint4*>(src + 16));
    } else {
      lf.a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  wave_sync_lds();                                            // reads done before the region is reused
#pragma unroll
  for (int t = 0; t < 4; ++t)
    lf.sc[t] = t < NT ? __uint_as_float((uint32_t)(127 + ct[t < NT ? t : 0] - 4 * G) << 23) : 0.f;
}

__device__ __forceinline__ void tile_mfma(TileAcc& acc, const QFrag& f, const v8i& b) {
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    acc.d[hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.a[hg], b, zero, 0, 0, 0, 0, 0, 0);
  }
}

__device__ __forceinline__ v4f lin_mfma(const LinFrag& lf, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lf.a, b, zero, 0, 0, 0, 0, 0, 0);
}

// This lane's 16 heads of one tile: sum of (w/2) |d| in a fixed order.  Its
// share of the linear half (the piece output row it holds for the token, times
// LinFrag::sc) is added right after, by the caller.
__device__ __forceinline__ float tile_epilogue(const QFrag& f, const TileAcc& acc) {
  float part = 0.f;
#pragma unroll
  for (int hg = 0; hg < 4; ++hg)
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(f.w[hg * 4 + i], fabsf(acc.d[hg][i]), part);
  return part;
}

// Reduce four per-tile partials over the lane groups and transpose, so that
// each lane returns the complete sum of position lane_pos(lane).
__device__ __forceinline__ float reduce_block(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float z = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float y = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(y), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Scores of one block for NT tokens: out[j] is token j's score at position
// lane_pos(lane).  Work items (token, tile) are issued token-fastest and
// pipelined two deep.  `bop(tl)` gives tile tl's B operand; it is asked for
// one tile ahead, so when it reads LDS the read is covered by a tile of MFMAs
// and only two tiles' operands are live.
template <int NT, typename BOp>
__device__ __forceinline__ void block_scores_with(const QFrag* f, const LinFrag& lf, BOp&& bop, float ks,
                                                  float* out) {
  constexpr int NI = 4 * NT;
  float part[NT][4];
  TileAcc acc[2];
  v8i b[2];
  b[0] = bop(0);
  b[1] = bop(1);
  if constexpr (NT == 1) {
    v4f lin[2];
    lin[0] = lin_mfma(lf, b[0]);
    tile_mfma(acc[0], f[0], b[0]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + 1 < NI) {
        const int tn = i + 1;
        if (tn >= 1 && tn + 1 < 4) b[(tn + 1) & 1] = bop(tn + 1);
        lin[tn & 1] = lin_mfma(lf, b[tn & 1]);
        tile_mfma(acc[(i + 1) & 1], f[0], b[tn & 1]);
      }
      part[0][i] = fmaf(lin[i & 1][0], lf.sc[0], tile_epilogue(f[0], acc[i & 1]));
    }
  } else {
    // the linear MFMA of a tile goes with its last token's MFMAs; its terms are
    // added once that token's epilogue is done (same operation order per token)
    v4f lin;
    tile_mfma(acc[0], f[0], b[0]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + 1 < NI) {
        const int tn = (i + 1) / NT;
        if ((i + 1) % NT == 0 && tn >= 1 && tn + 1 < 4) b[(tn + 1) & 1] = bop(tn + 1);
        if ((i + 1) % NT == NT - 1) lin = lin_mfma(lf, b[tn & 1]);
        tile_mfma(acc[(i + 1) & 1], f[(i + 1) % NT], b[tn & 1]);
      }
      const int t = i % NT, tl = i / NT;
      part[t][tl] = tile_epilogue(f[t], acc[i & 1]);
      if (t == NT - 1) {
#pragma unroll
        for (int u = 0; u < NT; ++u) part[u][tl] = fmaf(lin[u], lf.sc[u], part[u][tl]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j)
    out[j] = reduce_block(part[j][0], part[j][1], part[j][2], part[j][3]) * ks;
}

template <int NT>
__device__ __forceinline__ void block_scores(const QFrag* f, const LinFrag& lf, const KBlock& kb, float* out) {
  block_scores_with<NT>(f, lf, [&](int tl) { return kb.b[tl]; }, kb.ks, out);
}

// Tile tl's B operand straight from a staged block in LDS.
__device__ __forceinline__ v8i lds_tile(const uint8_t* slot, int tl, int lane) {
  const int c = lane & 15, G = lane >> 4;
  const int r = tl * 16 + c;
  const uint8_t* row = slot + r * kHeadDim;
  return pack8(*reinterpret_cast<const uint4*>(row + ((G ^ (r & 7)) << 4)),
               *reinterpret_cast<const uint4*>(row + (((4 + G) ^ (r & 7)) << 4)));
}

// ------------------------------------------------------ LDS staging --
// K blocks reach the MFMA operands through LDS: global loads are contiguous
// (8 lanes per 128-byte code row, whole lines per instruction), while the
// operand layout wants 16 rows x 64 bytes per load, which halves the lines
// per request and costs about a quarter of the achievable HBM rate.
// Same work split as above, but each K block is fetched once per work-group:
// the work-group copies it with contiguous 16-byte loads into LDS, two slots
// alternating, and every wave reads its MFMA operands from there.  The 16-byte
// chunk j of code row r sits at chunk (j ^ (r & 7)) of that row, so the
// MFMA-layout reads (16 rows, one chunk each, per lane group) hit distinct
// banks.
template <int NW>
struct StageRegs {
  static constexpr int kChunks = kBlockBytes / 16;                  // 528
  static constexpr int kPerThread = (kChunks + NW * 64 - 1) / (NW * 64);
  uint4 v[kPerThread];
  uint32_t mask;   // all ones for a block in the table, else 0 (stored as zeros)
};

// Offset past every block: a buffer load from it returns zeros and moves no data.
constexpr int kPastBlock = 0x10000;

template <int NW>
__device__ __forceinline__ int stage_src(int ci) {
  // LDS chunk ci <- global byte offset
  if (ci < kCodeBytes / 16) {
    const int r = ci >> 3, slot = ci & 7;
    return r * kHeadDim + ((slot ^ (r & 7)) << 4);
  }
  return ci << 4;                                                    // scales, unswizzled
}

// Every thread issues the same number of loads from a valid block address (in
// the last round the threads past the block's 528 chunks re-read one of its
// scale chunks), so no load sits behind a branch: a branch around a load makes
// the compiler wait for every load in flight at the next use, which would
// drain the prefetch.  A block absent from the table is read from block 0 and
// stored as zeros.  (Plain loads here: the range-checked buffer loads that the
// decode staging uses made prefill scoring ~3% slower, 1619-1647 against
// 1666-1701 us on 8192 tokens over 32K, alternated on one box.)
template <int NW>
__device__ __forceinline__ void stage_load(StageRegs<NW>& st, const uint8_t* __restrict__ base,
                                           bool valid) {
  constexpr int kC = StageRegs<NW>::kChunks;
#pragma unroll
  for (int u = 0; u < StageRegs<NW>::kPerThread; ++u) {
    int ci = threadIdx.x + u * NW * 64;
    if (u == StageRegs<NW>::kPerThread - 1 && (kC % (NW * 64)) != 0)
      ci = ci < kC ? ci : kC - 16 + (threadIdx.x & 15);
    st.v[u] = *reinterpret_cast<const uint4*>(base + stage_src<NW>(ci));
  }
  st.mask = valid ? 0xffffffffu : 0u;
}

template <int NW>
__device__ __forceinline__ void stage_store(const StageRegs<NW>& st, uint8_t* slot) {
#pragma unroll
  for (int u = 0; u < StageRegs<NW>::kPerThread; ++u) {
    const int ci = threadIdx.x + u * NW * 64;
    const uint4 x = make_uint4(st.v[u].x & st.mask, st.v[u].y & st.mask, st.v[u].z & st.mask,
                               st.v[u].w & st.mask);
    if (ci < StageRegs<NW>::kChunks) *reinterpret_cast<uint4*>(slot + (ci << 4)) = x;
  }
}

__device__ __forceinline__ void lds_kblock(KBlock& kb, const uint8_t* slot, int lane) {
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) kb.b[tl] = lds_tile(slot, tl, lane);
  kb.ks = *reinterpret_cast<const float*>(slot + kCodeBytes + lane_pos(lane) * 4);
}

// One wave stages a whole block: 528 16-byte chunks, 9 per lane (in the last
// round lanes 16-63 load from past the block, which fetches nothing), so every
// lane issues the same loads.  A block absent from the table or past the
// wave's run is loaded with `bytes` = 0: zeros, and no data moved.
struct WaveStage {
  uint4 v[9];
};

// The K stream of a decode batch is read once, so its loads are non-temporal
// (streamed past the caches): 59% -> 64.5% of the HBM peak on 8 x 128K rows.
__device__ __forceinline__ void wave_stage_load(WaveStage& st, const uint8_t* __restrict__ base,
                                                int bytes, int lane) {
  const __amdgpu_buffer_rsrc_t rs = byte_rsrc(base, bytes);
#pragma unroll
  for (int u = 0; u < 9; ++u) {
    const int off = u < 8 ? stage_src<1>(lane + 64 * u) : (lane < 16 ? (512 + lane) << 4 : kPastBlock);
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kLoadStream);
    st.v[u] = make_uint4(x[0], x[1], x[2], x[3]);
  }
}

__device__ __forceinline__ void wave_stage_store(const WaveStage& st, uint8_t* slot, int lane) {
#pragma unroll
  for (int u = 0; u < 9; ++u) {
    const int ci = lane + 64 * u;
    if (u < 8 || lane < 16) *reinterpret_cast<uint4*>(slot + (ci << 4)) = st.v[u];
  }
}

// ------------------------------------------------------------- decode --
// One query token per work-group; the work-group covers `chunk_blocks`
// consecutive 64-position blocks of its causal range, split into four
// consecutive runs, one per wave.  Each wave keeps the loads of its next NB-1
// blocks in flight in registers and passes the current block through its own
// LDS slot (`lds`: 4 * kBlockBytes) into the MFMA layout.
#ifndef IDX_DECODE_RING
#define IDX_DECODE_RING 2
#endif
#ifndef IDX_PREFILL_TPW
#define IDX_PREFILL_TPW 2
#endif
#ifndef IDX_PREFILL_MAX_CHUNK
#define IDX_PREFILL_MAX_CHUNK 64
#endif
#ifndef IDX_DECODE_WAVES_PER_EU
#define IDX_DECODE_WAVES_PER_EU 2
#endif

constexpr int kScoreThreads = 256;              // four waves, both work splits
constexpr int kPrefillTPW = IDX_PREFILL_TPW;    // query tokens per wave (prefill)
constexpr int kPrefillTM = 4 * kPrefillTPW;     // query tokens per work-group (prefill)
constexpr int kPrefillWin = (IDX_PREFILL_MAX_CHUNK + 63) / 64;   // block-id registers per lane (prefill)
static_assert(IDX_PREFILL_MAX_CHUNK >= 4 && IDX_PREFILL_MAX_CHUNK <= 256, "prefill chunk of 4..256 blocks");
constexpr int kLinScratch = 4096;                // LDS per wave for make_lin
constexpr int kPrefillLds = 2 * kBlockBytes + 4 * kLinScratch;
constexpr int kScoreLds = 4 * kBlockBytes;
static_assert(kScoreLds >= kPrefillLds && kBlockBytes >= kLinScratch, "LDS layout");

// This step's new K rows, for scoring kernels that write them into the cache
// themselves (decode batches of an F layer): row i of `k` belongs to query
// token i and goes to slots[i].
struct NewRows {
  const uint16_t* k;
  int64_t stride;
  const int64_t* slots;
  uint8_t* cache;      // the scored cache, writable
  int64_t num_slots;
};

// Requests with at most this many new tokens get their new rows written by
// the decode scoring kernel (a wave quantises the rows its blocks hold).
constexpr int kMaxFusedRows = 4;

// `ident`: token t is request t (every request has exactly one new token),
// which the host knows; the block-table slice of a full chunk is then read
// at once, in parallel with the request metadata.  With SPEC (the decode
// rows of a mixed batch, decodes first) request t's slice is read alongside
// the token lookup and kept if the lookup finds request t.
// Returns the token's causal count n, or -1 when the chunk holds none of its
// positions (then every wave of the work-group returns -1).
template <int NB, bool FK, bool SPEC = false>
__device__ __forceinline__ int decode_body(int bx, int t, const uint8_t* __restrict__ q8,
                                           const float* __restrict__ w, const CacheArgs& cache,
                                           const BatchArgs& b, float* __restrict__ logits,
                                           int64_t ld, int chunk_blocks, bool ident, uint8_t* lds,
                                           const NewRows& nk, float* __restrict__ samp) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
  const int lb0 = bx * chunk_blocks;
  const int per_full = chunk_blocks / 4;        // chunk_blocks is a multiple of 4
  const int lb_full = lb0 + wave * per_full + lane;
  int bt_full = -1;                             // raw id; checked only once it is needed
  const bool spec = SPEC && !ident && t < b.num_reqs;
  if ((ident || spec) && lane < per_full)
    bt_full = b.bt[(int64_t)t * b.bt_stride + min(lb_full, (int)b.bt_stride - 1)];
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
  load_q(f[0], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);  // first used by the MFMAs
  const int n = tp.n;
  if (lb0 * kBlock >= n) return -1;
  const int nblk = min(chunk_blocks, (n - lb0 * kBlock + kBlock - 1) / kBlock);
  const int per = (nblk + 3) / 4;
  const int mine = max(0, min(per, nblk - wave * per));        // blocks of this wave (<= 16)
  if (mine == 0) return n;
  const int lp = lane_pos(lane);
  auto blk = [&](int j) { return lb0 + wave * per + j; };
  float* out = logits + (size_t)t * ld;
  // the row's sampled scores also go to their compact copy (see sample_pos)
  float* srow = samp ? samp + (size_t)t * kMaxSample : nullptr;
  const int sS = sample_stride(n), sSh = 31 - __clz(sS);
  auto emit = [&](int j, float v) {
    const int s = blk(j) * kBlock + lp;
    const bool in = j < mine && s < n;
    if (in) out[s] = v;
    if (srow != nullptr) {
      const int sj = s >> sSh;
      if (in && (s & (sS - 1)) == ((37 * sj + 11) & (sS - 1))) srow[sj] = v;
    }
  };
  if (cache.num_blocks == 0) {                  // no K at all: every score is 0
    for (int j = 0; j < mine; ++j) emit(j, 0.f);
    return n;
  }
  // lane j holds the physical block of this wave's j-th block, so no K load
  // waits on a block-table load
  int pbl;
  if ((ident || (spec && tp.r == t)) && nblk == chunk_blocks)
    pbl = (lane < per_full && lb_full < b.bt_stride && bt_full >= 0 && bt_full < cache.num_blocks)
              ? bt_full : -1;
  else
    pbl = lane < mine ? (int)phys_block(b, cache, tp.r, blk(lane)) : -1;
  // block j of the run (j <= mine + NB - 2 < 64); past the run it loads nothing
  auto stage = [&](WaveStage& st, int j) {
    const int pb = __builtin_amdgcn_readlane(pbl, j);
    wave_stage_load(st, cache.data + (int64_t)max(pb, 0) * kBlockBytes,
                    (j < mine && pb >= 0) ? kBlockBytes : 0, lane);
  };
  uint8_t* slot = lds + wave * kBlockBytes;

  // Every iteration issues one block's loads (past the last block they fetch
  // nothing), so the loop body has no branch around a load.
  const int iters = (mine + NB - 1) / NB * NB;
  WaveStage ring[NB];
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) stage(ring[u], u);
  // the linear half's pieces, built in the wave's slot while the first loads
  // are in flight
  LinFrag lf;
  make_lin<1>(lf, f, slot, lane);

  // New rows of this token's request that fall in this wave's blocks and in
  // its causal range (positions len-nq .. p_t): quantised here, patched into
  // the staged block below, and the token's own row written to the cache.  A
  // row is patched only where its slot is the block-table slot of its
  // position; elsewhere the cache's contents are scored.
  uint32_t fcode[kMaxFusedRows];
  uint32_t fscale[kMaxFusedRows];
  int fpos0 = 0, nfix = 0;
  if (FK) {
    const int newlo = tp.len - tp.nq;
    const int lo = max(newlo, blk(0) * kBlock);
    const int hi = min(n - 1, (blk(mine - 1) + 1) * kBlock - 1);
    nfix = min(kMaxFusedRows, max(0, hi - lo + 1));
    fpos0 = lo;
#pragma unroll
    for (int i = 0; i < kMaxFusedRows; ++i) {
      fcode[i] = 0u;
      fscale[i] = 0u;
      if (i < nfix) {
        const int P = lo + i;
        const int row = tp.q0 + (P - newlo);
        const uint2 v = *reinterpret_cast<const uint2*>(nk.k + (int64_t)row * nk.stride + (lane & 31) * 4);
        const int64_t want = nk.slots[row];
        int e;
        const uint32_t code = quant_row_lane(v, &e);
        const uint32_t sc = __float_as_uint(pow2f(e));
        const int pb = __builtin_amdgcn_readlane(pbl, P / kBlock - blk(0));
        const bool patch = pb >= 0 && want == (int64_t)pb * kBlock + P % kBlock;
        fcode[i] = code;
        fscale[i] = patch ? sc : 0xFFFFFFFFu;   // all ones: leave the row as the cache has it
        if (row == t && want >= 0 && want < nk.num_slots) {   // the token's own row: to the cache
          uint8_t* cb = nk.cache + (want / kBlock) * kBlockBytes;
          if (lane < 32) *reinterpret_cast<uint32_t*>(cb + (want % kBlock) * kHeadDim + lane * 4) = code;
          if (lane == 0) *reinterpret_cast<uint32_t*>(cb + kCodeBytes + (want % kBlock) * 4) = sc;
        }
      }
    }
  }

  for (int j0 = 0; j0 < iters; j0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u;
      stage(ring[(u + NB - 1) % NB], j + NB - 1);
      __builtin_amdgcn_sched_barrier(0);        // nothing that needs block j moves above these loads
      wave_stage_store(ring[u], slot, lane);
      if (FK) {
#pragma unroll
        for (int i = 0; i < kMaxFusedRows; ++i) {
          const int P = fpos0 + i;
          if (i < nfix && fscale[i] != 0xFFFFFFFFu && P / kBlock == blk(j)) {
            const int rr = P % kBlock;
            if (lane < 32)
              *reinterpret_cast<uint32_t*>(slot + rr * kHeadDim + (((lane >> 2) ^ (rr & 7)) << 4) +
                                           (lane & 3) * 4) = fcode[i];
            if (lane == 0) *reinterpret_cast<uint32_t*>(slot + kCodeBytes + rr * 4) = fscale[i];
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      KBlock kb;
      lds_kblock(kb, slot, lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // reads done before the slot is rewritten
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float v;
      block_scores<1>(f, lf, kb, &v);
      emit(j, v);
    }
  }
  return n;
}

// ------------------------------------------------------------ kernels --
// Work-groups reach the XCDs round-robin in dispatch order (blockIdx.x
// fastest).  Each one takes its (chunk, row) from that order with the row
// fastest, so the chunks of one row -- whose costs differ: causal rows end
// early, a request's later chunks can be empty -- are spread over every XCD
// instead of chunk c always landing on XCD c mod 8.
__device__ __forceinline__ void xcd_spread(int* chunk, int* row) {
  const int L = blockIdx.y * gridDim.x + blockIdx.x;
  *row = L % gridDim.y;
  *chunk = L / gridDim.y;
}


// ----------------------------------------------------- prefill groups --
// Prefill groups are numbered across the batch: request r holds
// ceil(m_r / kPrefillTM) groups, m_r = its tokens at or above tok_lo (the
// first of them starting its first group), so ceil(P / kPrefillTM) + num_reqs
// groups cover any batch with P such tokens, and requests without prefill
// tokens (the decodes of a mixed batch) take no work-groups.  Every wave finds
// its group's request with a scan of the per-request group counts, 256
// requests per round of loads.
struct PrefillGroup {
  int r;    // request
  int q0;   // its first token (batch index), qsl[r]
  int nq;   // its tokens, qsl[r+1] - qsl[r]
  int len;  // its positions, seq_lens[r]
  int t0;   // first token of the group (batch index)
  int nt;   // tokens in the group, 1..kPrefillTM
};

__device__ __forceinline__ bool prefill_group(const BatchArgs& b, int G, int tok_lo, int gpr,
                                              PrefillGroup* pg) {
  constexpr int TM = kPrefillTM, U = 4;
  if (gpr > 0) {                                // per-request numbering: gpr groups per request
    const int r = G / gpr, g = G % gpr;
    if (r >= b.num_reqs) return false;
    pg->r = r;
    pg->q0 = b.qsl[r];
    pg->nq = b.qsl[r + 1] - pg->q0;
    pg->len = b.seq_lens[r];
    pg->t0 = pg->q0 + g * TM;
    pg->nt = min(TM, pg->nq - g * TM);
    return pg->nt > 0 && pg->t0 + pg->nt > tok_lo;
  }
  const int lane = threadIdx.x & 63;
  int base = 0;                                 // groups of the requests already passed
  for (int r0 = 0; r0 < b.num_reqs; r0 += 64 * U) {
    int lo[U], hi[U], len[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {               // every load of the round first
      const int r = r0 + 64 * u + lane;
      lo[u] = r < b.num_reqs ? b.qsl[r] : 0;
      hi[u] = r < b.num_reqs ? b.qsl[r + 1] : 0;
      len[u] = r < b.num_reqs ? b.seq_lens[r] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int l = max(lo[u], tok_lo);
      const int cnt = hi[u] > l ? (hi[u] - l + TM - 1) / TM : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const int total = __shfl(incl, 63, 64);
      if (G < base + total) {
        const uint64_t past = __ballot(G < base + incl);
        const int L = __ffsll((unsigned long long)past) - 1;
        const int excl = __builtin_amdgcn_readlane(incl - cnt, L);
        const int lL = __builtin_amdgcn_readlane(l, L);
        const int hL = __builtin_amdgcn_readlane(hi[u], L);
        pg->r = r0 + 64 * u + L;
        pg->q0 = __builtin_amdgcn_readlane(lo[u], L);
        pg->nq = hL - pg->q0;
        pg->len = __builtin_amdgcn_readlane(len[u], L);
        pg->t0 = lL + (G - base - excl) * TM;
        pg->nt = min(TM, hL - pg->t0);
        return true;
      }
      base += total;
    }
  }
  return false;
}

// Groups the prefill split launches for P tokens at or above tok_lo (at most
// one partial group per request that holds such tokens).
inline int64_t prefill_groups_bound(int64_t P, int num_reqs) {
  return (P + kPrefillTM - 1) / kPrefillTM + std::min<int64_t>(num_reqs, P);
}

// Prefill chunk: halved from the maximum until the grid holds `target`
// prefill work-groups, down to 4 blocks.  The target is 1024 (two per
// work-group slot): smaller chunks add more per-work-group set-up than they
// balance.  When a mixed launch's decode work-groups alone fill every slot,
// the target is 2048, so that short prefill work-groups fill in around them.
inline int prefill_chunk_blocks(const BatchArgs& b, int64_t groups, bool fill_around) {
  const int64_t target = fill_around ? 2048 : 1024;
  int cb = IDX_PREFILL_MAX_CHUNK;
  while (cb > 4 && groups * ((b.max_seq_len + cb * kBlock - 1) / (cb * kBlock)) < target) cb >>= 1;
  return cb;
}


}  // namespace
}  // namespace idx

// Lightning-indexer scores on gfx950 matrix cores.
//
//   I[t, s] = ks[s] * sum_h w[t, h] * max(0, q8[t, h, :] . k8[s, :])
//
// (IndexCache blog post: SparseAttnIndexer / Indexer.forward -- 64 fp8 query
// heads share one fp8 K per position, folded fp32 weights; the score's form is
// the DSA lightning indexer's.)
//
// The head dot products are one v_mfma_f32_16x16x128_f8f6f4 per 16 heads x 16
// positions: A = q rows of 16 heads (128 fp8 each), B = 16 K rows.  The MFMA
// leaves D[head 4*(lane/16)+i][position lane%16] in lane `lane`, register i,
// so the ReLU and the head weighting run in registers right after the MFMA,
// each lane summing its 16 heads, and two cross-lane adds finish the 64-head
// sum.  Both operands use the same byte->k assignment (lane group G = lane/16
// holds k in [16G, 16G+16) and [64+16G, 64+16G+16)), so the contraction covers
// all 128 dimensions whatever the hardware's own k order is.
//
// Every kernel computes a score with exactly this sequence of operations, so
// all kernels and all entry points give bit-identical scores.

#include "common.hpp"
#include "launch.hpp"

namespace idx {
namespace {

// One token's q as four A operands (16 heads each) plus this lane's 16 weights
// w[16*hg + 4*(lane/16) + i] in w[4*hg + i].
struct QFrag {
  v8i a[4];
  float w[16];
};

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
    f.w[hg * 4 + 0] = wv.x; f.w[hg * 4 + 1] = wv.y;
    f.w[hg * 4 + 2] = wv.z; f.w[hg * 4 + 3] = wv.w;
  }
}

__device__ __forceinline__ void zero_q(QFrag& f) {
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    f.a[hg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) f.w[hg * 4 + i] = 0.f;
  }
}

// Head-weighted ReLU sum for the 16 positions of one K tile; every lane of a
// column (lane % 16) returns the same value.
__device__ __forceinline__ float tile_score(const QFrag& f, const v8i& b) {
  float part = 0.f;
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.a[hg], b, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(f.w[hg * 4 + i], fmaxf(acc[i], 0.f), part);
  }
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  return part;
}

// The four 16-position tiles of one 64-position block: B operands and scales.
struct KBlock {
  v8i b[4];
  float ks[4];
};

__device__ __forceinline__ void load_kblock(KBlock& kb, const uint8_t* __restrict__ base,
                                            int lane) {
  const int c = lane & 15, G = lane >> 4;
  if (base == nullptr) {
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) {
      kb.b[tl] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      kb.ks[tl] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const uint8_t* row = base + (tl * 16 + c) * kHeadDim;
    kb.b[tl] = pack8(*reinterpret_cast<const uint4*>(row + 16 * G),
                     *reinterpret_cast<const uint4*>(row + 64 + 16 * G));
    kb.ks[tl] = *reinterpret_cast<const float*>(base + kCodeBytes + (tl * 16 + c) * 4);
  }
}

__device__ __forceinline__ const uint8_t* block_base(const BatchArgs& b, const CacheArgs& c, int r,
                                                     int lb) {
  const int64_t pb = phys_block(b, c, r, lb);
  return pb < 0 ? nullptr : c.data + pb * kBlockBytes;
}

// ------------------------------------------------------------- decode --
// One query token per work-group; the work-group covers `chunk_blocks`
// consecutive 64-position blocks of its causal range and its four waves take
// every fourth block.  Each wave keeps the next block's loads in flight while
// it scores the current one.
__global__ __launch_bounds__(256) void score_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    float* __restrict__ logits, int64_t ld, int chunk_blocks) {
  const int t = blockIdx.y;
  const TokenPos tp = token_pos(b, t);
  const int n = tp.n;
  const int lb0 = blockIdx.x * chunk_blocks;
  if (lb0 * kBlock >= n) return;
  const int nblk = min(chunk_blocks, (n - lb0 * kBlock + kBlock - 1) / kBlock);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;

  QFrag f;
  load_q(f, q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
  float* out = logits + (size_t)t * ld;

  KBlock cur, nxt;
  if (wave < nblk) load_kblock(cur, block_base(b, cache, tp.r, lb0 + wave), lane);
  for (int bi = wave; bi < nblk; bi += 4) {
    const bool more = bi + 4 < nblk;
    if (more) load_kblock(nxt, block_base(b, cache, tp.r, lb0 + bi + 4), lane);
    const int sb = (lb0 + bi) * kBlock;
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) {
      const float v = tile_score(f, cur.b[tl]) * cur.ks[tl];
      const int s = sb + tl * 16 + c;
      if (G == 0 && s < n) out[s] = v;
    }
    if (more) cur = nxt;
  }
}

// ------------------------------------------------------------ prefill --
// A work-group takes 4*TPW consecutive query tokens of one request (TPW per
// wave) and `chunk_blocks` blocks of positions; all four waves walk the same
// blocks, so each K tile is fetched from HBM once per work-group and reused
// from the caches by the other waves.
template <int TPW>
__global__ __launch_bounds__(256) void score_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ w, CacheArgs cache, BatchArgs b,
    float* __restrict__ logits, int64_t ld, int chunk_blocks, int groups_per_req) {
  constexpr int TM = 4 * TPW;
  const int r = blockIdx.y / groups_per_req;
  const int g = blockIdx.y % groups_per_req;
  if (r >= b.num_reqs) return;
  const int q0 = b.qsl[r];
  const int nq = b.qsl[r + 1] - q0;
  const int tb = g * TM;
  if (tb >= nq) return;
  const int L = b.seq_lens[r];
  auto count = [&](int i) {  // causal positions of the request's i-th new token
    int n = L - nq + i + 1;
    n = n < 0 ? 0 : n;
    return n > b.max_seq_len ? b.max_seq_len : n;
  };
  const int n_max = count(min(tb + TM, nq) - 1);
  const int lb0 = blockIdx.x * chunk_blocks;
  if (lb0 * kBlock >= n_max) return;
  const int nblk = min(chunk_blocks, (n_max - lb0 * kBlock + kBlock - 1) / kBlock);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;

  QFrag f[TPW];
  int nt[TPW];
  float* out[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int i = tb + wave * TPW + j;
    const int t = q0 + i;
    if (i < nq && t >= 0 && t < b.num_tokens) {
      load_q(f[j], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
      nt[j] = count(i);
      out[j] = logits + (size_t)t * ld;
    } else {
      zero_q(f[j]);
      nt[j] = 0;
      out[j] = logits;
    }
  }

  KBlock cur, nxt;
  load_kblock(cur, block_base(b, cache, r, lb0), lane);
  for (int bi = 0; bi < nblk; ++bi) {
    const bool more = bi + 1 < nblk;
    if (more) load_kblock(nxt, block_base(b, cache, r, lb0 + bi + 1), lane);
    const int sb = (lb0 + bi) * kBlock;
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) {
      const int s = sb + tl * 16 + c;
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const float v = tile_score(f[j], cur.b[tl]) * cur.ks[tl];
        if (G == 0 && s < nt[j]) out[j][s] = v;
      }
    }
    if (more) cur = nxt;
  }
}

constexpr int kDecodeChunkBlocks = 16;   // 1024 positions per work-group
constexpr int kPrefillTPW = 2;

int prefill_chunk_blocks(const BatchArgs& b) {
  // aim for a few thousand work-groups; never more blocks than the longest row needs
  const int gpr = (b.max_query_len + 4 * kPrefillTPW - 1) / (4 * kPrefillTPW);
  const int64_t groups = (int64_t)gpr * b.num_reqs;
  int cb = 32;
  while (cb > 4 && groups * ((b.max_seq_len + cb * kBlock - 1) / (cb * kBlock)) < 2048) cb >>= 1;
  return cb;
}

}  // namespace

hipError_t launch_score(const uint8_t* q8, const float* w, const CacheArgs& cache,
                        const BatchArgs& b, float* logits, int64_t ld, hipStream_t stream) {
  if (b.num_tokens == 0 || b.max_seq_len == 0) return hipSuccess;
  if (b.max_query_len <= 1) {
    const int cb = kDecodeChunkBlocks;
    const int chunks = (b.max_seq_len + cb * kBlock - 1) / (cb * kBlock);
    const dim3 grid((unsigned)chunks, (unsigned)b.num_tokens);
    hipLaunchKernelGGL(score_decode_kernel, grid, dim3(256), 0, stream, q8, w, cache, b, logits,
                       ld, cb);
  } else {
    const int cb = prefill_chunk_blocks(b);
    const int gpr = (b.max_query_len + 4 * kPrefillTPW - 1) / (4 * kPrefillTPW);
    const int chunks = (b.max_seq_len + cb * kBlock - 1) / (cb * kBlock);
    const dim3 grid((unsigned)chunks, (unsigned)(gpr * b.num_reqs));
    hipLaunchKernelGGL(score_prefill_kernel<kPrefillTPW>, grid, dim3(256), 0, stream, q8, w, cache,
                       b, logits, ld, cb, gpr);
  }
  return hipGetLastError();
}

}  // namespace idx

// The FP4 indexer K cache: quantise-and-scatter and scoring.
//
// The pages name this variant of the cache (IndexCache blog post: the
// use_fp4_cache argument SparseAttnIndexer.forward_cuda passes to the op) but
// not its format.  The format here is the OCP MX one that gfx950's scaled
// matrix cores take as an operand without any conversion:
//
//  * K row of 128 values = four groups of 32 dims; group g has a
//    power-of-two scale 2^e, e the smallest integer with
//    max(amax_g, 1e-4) <= 6 * 2^e (E8M0 byte e + 127), and each value the
//    E2M1 code of x / 2^e (nearest, ties to even, sign kept);
//  * block of 64 positions, 4352 bytes:
//      codes   g*1024 + p*16 + i      dims 32g+2i (bits 0-3), 32g+2i+1 (bits 4-7)
//      scales  4096 + g*64 + (p%16)*4 + p/16
//    so a 16-position tile of group g is 256 contiguous bytes, and each lane
//    finds its position's four tiles' scale bytes in one dword.
//
// Scores: I[t, s] = sum_h w[t, h] * max(0, sum_d q8[t, h, d] * c[s, d] * 2^e[s, d/32]).
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = the fp8 q rows (the layout of
// the FP8 path: lane group G holds dims 16G.. and 64+16G..), B = fp4 codes
// (lane group G holds dims 32G..32G+31, low nibble first) and B's scale
// operand = the codes' E8M0 bytes (the k block of 32 dims G takes its scale
// from lane group G; op_sel picks the tile's byte of the dword).  The ReLU
// split, the linear half's pieces, the epilogue and the lane transpose are
// the FP8 path's (score_device.hpp); the K scale is inside the MFMA, so no
// per-position factor remains.

#include "common.hpp"
#include "launch.hpp"
#include "score_device.hpp"
#include "fp4_device.hpp"

#ifndef IDX_FP4_DECODE_RING
#define IDX_FP4_DECODE_RING 4
#endif

namespace idx {
namespace {

// 32 lanes per row, lane q owns dims 4q..4q+3 (group q/8).
constexpr int kFp4QuantRows = 8;                 // rows per 256-thread work-group

__global__ __launch_bounds__(256) void quant_write_k_fp4_kernel(const uint16_t* __restrict__ k,
                                                                int64_t num_rows, int64_t stride,
                                                                const int64_t* __restrict__ slots,
                                                                uint8_t* __restrict__ cache,
                                                                int64_t num_slots) {
  const int64_t row = (int64_t)blockIdx.x * kFp4QuantRows + (threadIdx.x >> 5);
  const int q = threadIdx.x & 31;
  if (row >= num_rows) return;                   // the row's 32 lanes leave together
  const int64_t slot = slots[row];
  if (slot < 0 || slot >= num_slots) return;
  const uint2 v = *reinterpret_cast<const uint2*>(k + row * stride + q * 4);
  const uint32_t x[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
  uint32_t am = max(max(x[0] & 0x7FFFu, x[1] & 0x7FFFu), max(x[2] & 0x7FFFu, x[3] & 0x7FFFu));
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 32));
  const int e = fp4_exponent(am);
  const float s = pow2f(-e);
  const uint32_t codes = encode_e2m1(x[0], s) | (encode_e2m1(x[1], s) << 4) |
                         (encode_e2m1(x[2], s) << 8) | (encode_e2m1(x[3], s) << 12);
  const int64_t blk = slot / kBlock;
  const int p = (int)(slot % kBlock), g = q >> 3;
  uint8_t* base = cache + blk * kFp4BlockBytes;
  *reinterpret_cast<uint16_t*>(base + g * kFp4Plane + p * 16 + 2 * (q & 7)) = (uint16_t)codes;
  if ((q & 7) == 0) base[kFp4CodeBytes + g * 64 + (p & 15) * 4 + (p >> 4)] = (uint8_t)(e + 127);
}

// Prefill split: kPrefillTM consecutive query tokens of one request per
// work-group (kPrefillTPW per wave) over `chunk_blocks` blocks.  Every wave
// loads each block's operands itself (the four waves' loads of one block
// meet in the caches) and keeps NB-1 blocks in flight.
template <int NB>
__device__ __forceinline__ void fp4_prefill_body(int bx, int gy, const uint8_t* __restrict__ q8,
                                                 const float* __restrict__ w, const CacheArgs& cache,
                                                 const BatchArgs& b, float* __restrict__ logits,
                                                 int64_t ld, int chunk_blocks, int gpr, uint8_t* lds,
                                                 float* __restrict__ samp) {
  constexpr int TPW = kPrefillTPW;
  PrefillGroup pg;
  if (!prefill_group(b, gy, 0, gpr, &pg)) return;
  const int tb = pg.t0 - pg.q0;
  auto count = [&](int i) {
    int n = pg.len - pg.nq + i + 1;
    n = n < 0 ? 0 : n;
    return n > b.max_seq_len ? b.max_seq_len : n;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  QFrag f[TPW];
  int nt[TPW], tk[TPW], sS[TPW], sSh[TPW];
  int n_max = 0;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int i = tb + wave * TPW + j;
    const int t = pg.q0 + i;
    if (i < tb + pg.nt && t < b.num_tokens) {
      load_q(f[j], q8 + (size_t)t * kHeads * kHeadDim, w + (size_t)t * kHeads, lane);
      nt[j] = count(i);
      tk[j] = t;
    } else {
      zero_q(f[j]);
      nt[j] = 0;
      tk[j] = 0;
    }
    n_max = max(n_max, nt[j]);
    sS[j] = sample_stride(nt[j]);
    sSh[j] = 31 - __clz(sS[j]);
  }
  const int lb0 = bx * chunk_blocks;
  if (lb0 * kBlock >= n_max) return;            // nothing of this wave's tokens in the chunk
  const int nblk = min(chunk_blocks, (n_max - lb0 * kBlock + kBlock - 1) / kBlock);
  int pbl[kPrefillWin];
#pragma unroll
  for (int v = 0; v < kPrefillWin; ++v)
    pbl[v] = 64 * v + lane < nblk ? (int)phys_block(b, cache, pg.r, lb0 + 64 * v + lane) : -1;
  auto load = [&](KBlock4& kb, int j) {
    const int jc = min(j, 64 * kPrefillWin - 1);
    int v = pbl[0];
#pragma unroll
    for (int x = 1; x < kPrefillWin; ++x) v = (jc >> 6) == x ? pbl[x] : v;
    const int pb = __builtin_amdgcn_readlane(v, jc & 63);
    fp4_block_load<0>(kb, cache.data + (int64_t)max(pb, 0) * kFp4BlockBytes,
                      (j < nblk && pb >= 0) ? kFp4BlockBytes : 0, lane);
  };
  KBlock4 ring[NB];
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) load(ring[u], u);
  LinFrag lf;
  make_lin<TPW>(lf, f, lds + wave * kLinScratch, lane);
  const int lp = lane_pos(lane);
  const int iters = (nblk + NB - 1) / NB * NB;
  for (int j0 = 0; j0 < iters; j0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u;
      load(ring[(u + NB - 1) % NB], j + NB - 1);
      __builtin_amdgcn_sched_barrier(0);
      float v[TPW];
      fp4_block_scores<TPW>(f, lf, ring[u], v);
      if (j < nblk) {
        const int s = (lb0 + j) * kBlock + lp;
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj)
          fp4_emit(logits + (size_t)tk[jj] * ld, samp ? samp + (size_t)tk[jj] * kMaxSample : nullptr,
                   s, nt[jj], sS[jj], sSh[jj], v[jj]);
      }
    }
  }
}

#ifndef IDX_FP4_PREFILL_RING
#define IDX_FP4_PREFILL_RING 2
#endif

template <int NB>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(2)))
void score_fp4_decode_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ w,
                             CacheArgs cache, BatchArgs b, float* __restrict__ logits, int64_t ld,
                             int chunk_blocks, float* samp) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kLinScratch];
  int cx, ry;
  xcd_spread(&cx, &ry);
  fp4_decode_body<NB>(cx, ry, q8, w, cache, b, logits, ld, chunk_blocks,
                      b.num_reqs == b.num_tokens && b.max_query_len <= 1, lds, samp);
}

template <int NB>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(2)))
void score_fp4_prefill_kernel(const uint8_t* __restrict__ q8, const float* __restrict__ w,
                              CacheArgs cache, BatchArgs b, float* __restrict__ logits, int64_t ld,
                              int chunk_blocks, int gpr, float* samp) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kLinScratch];
  int cx, ry;
  xcd_spread(&cx, &ry);
  fp4_prefill_body<NB>(cx, ry, q8, w, cache, b, logits, ld, chunk_blocks, gpr, lds, samp);
}

}  // namespace

hipError_t launch_quant_write_k_fp4(const uint16_t* k, int64_t num_rows, int64_t stride,
                                    const int64_t* slots, uint8_t* cache, int64_t num_slots,
                                    hipStream_t stream) {
  const int64_t blocks = (num_rows + kFp4QuantRows - 1) / kFp4QuantRows;
  IDX_LAUNCH("quant_write_k_fp4_kernel", (quant_write_k_fp4_kernel), dim3((unsigned)blocks),
             dim3(256), stream, k, num_rows, stride, slots, cache, num_slots);
  return hipGetLastError();
}

hipError_t launch_score_fp4(const uint8_t* q8, const float* w, const CacheArgs& cache,
                            const BatchArgs& b, int64_t dec_tokens, float* logits, int64_t ld,
                            float* samp, hipStream_t stream) {
  if (b.num_tokens == 0 || b.max_seq_len == 0) return hipSuccess;
  if (b.max_query_len <= 1 || dec_tokens >= b.num_tokens) {
    const int cb = decode_chunk_blocks(b.max_seq_len, b.num_tokens);
    const int chunks = (b.max_seq_len + cb * kBlock - 1) / (cb * kBlock);
    IDX_LAUNCH("score_fp4_decode_kernel", (score_fp4_decode_kernel<IDX_FP4_DECODE_RING>),
               dim3((unsigned)chunks, (unsigned)b.num_tokens), dim3(kScoreThreads), stream, q8, w,
               cache, b, logits, ld, cb, samp);
    return hipGetLastError();
  }
  // every token with the prefill split (a mixed batch's decodes take a group each)
  const int64_t per_req = (int64_t)((b.max_query_len + kPrefillTM - 1) / kPrefillTM);
  const int64_t flat = prefill_groups_bound(b.num_tokens, b.num_reqs);
  const bool arith = per_req * b.num_reqs <= flat + flat / 4;
  const int gpr = arith ? (int)per_req : 0;
  const int64_t groups = arith ? per_req * b.num_reqs : flat;
  if (groups > 65535) return hipErrorInvalidConfiguration;      // grid y-extent
  const int pcb = prefill_chunk_blocks(b, groups, false);
  const int pchunks = (b.max_seq_len + pcb * kBlock - 1) / (pcb * kBlock);
  IDX_LAUNCH("score_fp4_prefill_kernel", (score_fp4_prefill_kernel<IDX_FP4_PREFILL_RING>),
             dim3((unsigned)pchunks, (unsigned)groups), dim3(kScoreThreads), stream, q8, w, cache, b,
             logits, ld, pcb, gpr, samp);
  return hipGetLastError();
}

}  // namespace idx

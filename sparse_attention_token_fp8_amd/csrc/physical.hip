// Logical -> physical top-k indices, once per index group.
//
// Page: vLLM API docs, vllm.v1.attention.backends.mla.index_group --
// SparseMLAIndexGroup.convert_logical_to_physical_topk / _convert_once turn a
// token's logical top-k (request positions) into global cache slots through the
// token's request, the block table and the block size, optionally returning the
// number of valid entries per row.  Here: slot = block * stride_rows +
// pos % block_size, -1 stays -1, and a position outside 0..p_t or a block
// outside the pool also gives -1.

#include "common.hpp"
#include "launch.hpp"
#include "topk_device.hpp"

namespace idx {
namespace {

// One work-group per token; each thread converts 8 consecutive entries (two
// 16-byte loads and stores when the row is 16-byte aligned), so the block-table
// reads of a row are all in flight together.  The row's first entries are
// loaded before the token's request is looked up, so the two round trips
// overlap; the valid count is summed with ballots (no block scan).  Rows are
// read and written once, with non-temporal loads and stores.  (Two or four
// tokens per work-group measured slower.)
constexpr int kPhysPer = 8;

__device__ __forceinline__ void phys_load(int* pos, const int32_t* __restrict__ in, int jb, int k,
                                          bool vec) {
  if (vec && jb + kPhysPer <= k) {
    typedef int i4v __attribute__((ext_vector_type(4)));
    const i4v a = __builtin_nontemporal_load(reinterpret_cast<const i4v*>(in + jb));
    const i4v d = __builtin_nontemporal_load(reinterpret_cast<const i4v*>(in + jb + 4));
    pos[0] = a[0]; pos[1] = a[1]; pos[2] = a[2]; pos[3] = a[3];
    pos[4] = d[0]; pos[5] = d[1]; pos[6] = d[2]; pos[7] = d[3];
  } else {
#pragma unroll
    for (int e = 0; e < kPhysPer; ++e) pos[e] = jb + e < k ? in[jb + e] : -1;
  }
}

// POW2: block_size is 1 << bs_shift, so an entry's block and offset are a
// shift and a mask instead of a division.  Every slot of the pool fits in 32
// bits (num_blocks * stride_rows <= INT32_MAX, checked on the host), so the
// per-entry arithmetic is 32-bit; only the request's block-table row is
// addressed in 64 bits, once.
template <bool POW2>
__global__ __launch_bounds__(256) void to_physical_kernel(const int32_t* __restrict__ logical,
                                                          int64_t ldl, BatchArgs b, CacheArgs c,
                                                          int block_size, int bs_shift, int k,
                                                          int64_t stride_rows,
                                                          int32_t* __restrict__ phys, int64_t ldp,
                                                          int32_t* __restrict__ valid) {
  constexpr int kStep = kThreads * kPhysPer;
  const int t = blockIdx.x;
  const int32_t* in = logical + (size_t)t * ldl;
  int32_t* out = phys + (size_t)t * ldp;
  const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  int pos[kPhysPer];
  phys_load(pos, in, (int)threadIdx.x * kPhysPer, k, vec);
  const TokenPos tp = token_pos_wave(b, t);
  const int32_t* __restrict__ btr = b.bt + (int64_t)tp.r * b.bt_stride;
  const int bt_n = (int)min(b.bt_stride, (int64_t)INT32_MAX);
  const int nb = (int)min(c.num_blocks, (int64_t)INT32_MAX);
  const uint32_t srow = (uint32_t)min(stride_rows, (int64_t)INT32_MAX);   // used only when nb > 0
  uint32_t cnt = 0;                             // valid entries of this wave (uniform)
  for (int j0 = 0; j0 < k; j0 += kStep) {
    const int jb = j0 + (int)threadIdx.x * kPhysPer;
    int32_t o[kPhysPer];
#pragma unroll
    for (int e = 0; e < kPhysPer; ++e) {
      o[e] = -1;
      const int p = pos[e];
      if (p >= 0 && p < tp.n) {
        const int lb = POW2 ? p >> bs_shift : p / block_size;
        const int off = POW2 ? p & (block_size - 1) : p - lb * block_size;
        if (lb < bt_n) {
          const int blk = btr[lb];
          if (blk >= 0 && blk < nb) o[e] = (int32_t)((uint32_t)blk * srow + (uint32_t)off);
        }
      }
      cnt += (uint32_t)__popcll(__ballot(jb + e < k && o[e] >= 0));
    }
    if (vec && jb + kPhysPer <= k) {
      typedef int i4o __attribute__((ext_vector_type(4)));
      const i4o o0 = {o[0], o[1], o[2], o[3]}, o1 = {o[4], o[5], o[6], o[7]};
      __builtin_nontemporal_store(o0, reinterpret_cast<i4o*>(out + jb));
      __builtin_nontemporal_store(o1, reinterpret_cast<i4o*>(out + jb + 4));
    } else {
#pragma unroll
      for (int e = 0; e < kPhysPer; ++e)
        if (jb + e < k) out[jb + e] = o[e];
    }
    if (j0 + kStep < k) phys_load(pos, in, jb + kStep, k, vec);
  }
  if (valid != nullptr) {
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t total = 0;
#pragma unroll
      for (int i = 0; i < kThreads / 64; ++i) total += part[i];
      valid[t] = (int32_t)total;
    }
  }
}

}  // namespace

hipError_t launch_topk_to_physical(const int32_t* logical, int64_t ldl, const BatchArgs& b,
                                   int block_size, int64_t num_blocks, int k, int64_t stride_rows,
                                   int32_t* physical, int64_t ldp, int32_t* valid,
                                   hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  CacheArgs c{nullptr, num_blocks};
  if ((block_size & (block_size - 1)) == 0)
    IDX_LAUNCH("to_physical_kernel", (to_physical_kernel<true>), dim3((unsigned)b.num_tokens),
               dim3(256), stream, logical, ldl, b, c, block_size,
               __builtin_ctz((unsigned)block_size), k, stride_rows, physical, ldp, valid);
  else
    IDX_LAUNCH("to_physical_kernel", (to_physical_kernel<false>), dim3((unsigned)b.num_tokens),
               dim3(256), stream, logical, ldl, b, c, block_size, 0, k, stride_rows, physical,
               ldp, valid);
  return hipGetLastError();
}

}  // namespace idx

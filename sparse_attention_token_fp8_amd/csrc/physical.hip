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

__global__ __launch_bounds__(256) void to_physical_kernel(const int32_t* __restrict__ logical,
                                                          int64_t ldl, BatchArgs b, CacheArgs c,
                                                          int block_size, int k,
                                                          int64_t stride_rows,
                                                          int32_t* __restrict__ phys, int64_t ldp,
                                                          int32_t* __restrict__ valid) {
  const int t = blockIdx.x;
  const TokenPos tp = token_pos(b, t);
  __shared__ uint32_t scratch[8];
  uint32_t cnt = 0;
  for (int j = threadIdx.x; j < k; j += kThreads) {
    const int pos = logical[(size_t)t * ldl + j];
    int32_t o = -1;
    if (pos >= 0 && pos < tp.n) {
      const int64_t blk = phys_block(b, c, tp.r, pos / block_size);
      if (blk >= 0) o = (int32_t)(blk * stride_rows + pos % block_size);
    }
    phys[(size_t)t * ldp + j] = o;
    cnt += o >= 0;
  }
  uint32_t total;
  (void)block_scan_excl<kThreads>(cnt, &total, scratch);
  if (valid && threadIdx.x == 0) valid[t] = (int32_t)total;
}

}  // namespace

hipError_t launch_topk_to_physical(const int32_t* logical, int64_t ldl, const BatchArgs& b,
                                   int block_size, int64_t num_blocks, int k, int64_t stride_rows,
                                   int32_t* physical, int64_t ldp, int32_t* valid,
                                   hipStream_t stream) {
  if (b.num_tokens == 0) return hipSuccess;
  CacheArgs c{nullptr, num_blocks};
  hipLaunchKernelGGL(to_physical_kernel, dim3((unsigned)b.num_tokens), dim3(256), 0, stream,
                     logical, ldl, b, c, block_size, k, stride_rows, physical, ldp, valid);
  return hipGetLastError();
}

}  // namespace idx

// fp8 (E4M3) quantisation with power-of-two scales: the K quantise-and-scatter
// into the paged cache, and the per-(token, head) q quantisation with the
// weight fold.
//
// Sources: IndexCache blog post (atomage.cn) -- the op body calls
// ops.indexer_k_quant_and_cache(k, kv_cache, slot_mapping, quant_block_size,
// scale_fmt); the "FP8 naive cache" snippet gives 128 code bytes plus one
// 4-byte fp32 scale per token; Indexer.forward quantises q per group of 128
// with ue8m0 scales and folds q_scale * softmax_scale * n_head^-0.5 into the
// weights.
//
// The quantiser itself (integer-only, see quant_device.hpp) is shared with the
// top-k planning kernel.

#include "common.hpp"
#include "launch.hpp"
#include "quant_device.hpp"

namespace idx {
namespace {

constexpr int kRowsPerBlock = 8;  // 32 lanes per 128-wide row, 256 threads

__global__ __launch_bounds__(256) void quant_write_k_kernel(const uint16_t* __restrict__ k,
                                                            int64_t num_rows, int64_t stride,
                                                            const int64_t* __restrict__ slots,
                                                            uint8_t* __restrict__ cache,
                                                            int64_t num_slots) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 5);
  const int lane = threadIdx.x & 31;
  if (row >= num_rows) return;                     // whole 32-lane group leaves together
  quant_write_row(k + row * stride, slots[row], cache, num_slots, lane);
}

__global__ __launch_bounds__(256) void quant_q_fold_kernel(const uint16_t* __restrict__ q,
                                                           const float* __restrict__ w_raw,
                                                           int64_t num_rows, float softmax_scale,
                                                           float head_norm, uint8_t* __restrict__ q8,
                                                           float* __restrict__ w_out,
                                                           float* __restrict__ qs_out) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 5);
  const int lane = threadIdx.x & 31;
  if (row >= num_rows) return;
  const uint2 v = *reinterpret_cast<const uint2*>(q + row * kHeadDim + lane * 4);
  int e;
  const uint32_t codes = quant_row_lane(v, &e);
  *reinterpret_cast<uint32_t*>(q8 + row * kHeadDim + lane * 4) = codes;
  if (lane == 0) {
    const float qs = pow2f(e);
    // ((w * q_scale) * softmax_scale) * n_head^-0.5, each product rounded to fp32
    float wf = __fmul_rn(w_raw[row], qs);
    wf = __fmul_rn(wf, softmax_scale);
    wf = __fmul_rn(wf, head_norm);
    w_out[row] = wf;
    if (qs_out) qs_out[row] = qs;
  }
}

// The same fold with 16 lanes per row and four rows per lane group, every
// load of a work-group issued before the first row is encoded, and the codes
// from the hardware E4M3 conversion (q 16-byte aligned).
constexpr int kFoldPass = 4;                    // rows per 16-lane group
constexpr int kFoldRows = 16 * kFoldPass;       // rows per 256-thread work-group

__global__ __launch_bounds__(256) void quant_q_fold16_kernel(const uint16_t* __restrict__ q,
                                                             const float* __restrict__ w_raw,
                                                             int64_t num_rows, float softmax_scale,
                                                             float head_norm, uint8_t* __restrict__ q8,
                                                             float* __restrict__ w_out,
                                                             float* __restrict__ qs_out) {
  const int lane = threadIdx.x & 15;
  const int64_t row0 = (int64_t)blockIdx.x * kFoldRows + (threadIdx.x >> 4);
  uint4 v[kFoldPass];
  float wr[kFoldPass];
#pragma unroll
  for (int p = 0; p < kFoldPass; ++p) {
    const int64_t row = row0 + 16 * p;
    const bool ok = row < num_rows;             // uniform over the 16 lanes of the row
    // q is read once and q8 written once per call: non-temporal (67% -> 75%
    // of the HBM peak on 8192 tokens x 64 heads)
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    u4v x = {0u, 0u, 0u, 0u};
    if (ok) x = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(q + row * kHeadDim + lane * 8));
    v[p] = make_uint4(x[0], x[1], x[2], x[3]);
    wr[p] = ok && lane == 0 ? w_raw[row] : 0.f;
  }
#pragma unroll
  for (int p = 0; p < kFoldPass; ++p) {
    const int64_t row = row0 + 16 * p;
    int e;
    const uint2 codes = quant_row_lane8_cvt(v[p], &e);
    if (row >= num_rows) continue;
    {
      typedef unsigned int u2v __attribute__((ext_vector_type(2)));
      u2v c2 = {codes.x, codes.y};
      __builtin_nontemporal_store(c2, reinterpret_cast<u2v*>(q8 + row * kHeadDim + lane * 8));
    }
    if (lane == 0) {
      const float qs = pow2f(e);
      float wf = __fmul_rn(wr[p], qs);
      wf = __fmul_rn(wf, softmax_scale);
      wf = __fmul_rn(wf, head_norm);
      w_out[row] = wf;
      if (qs_out) qs_out[row] = qs;
    }
  }
}

}  // namespace

hipError_t launch_quant_write_k(const uint16_t* k, int64_t num_rows, int64_t stride,
                                const int64_t* slots, uint8_t* cache, int64_t num_slots,
                                hipStream_t stream) {
  const int64_t blocks = (num_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  IDX_LAUNCH("quant_write_k_kernel", (quant_write_k_kernel), dim3((unsigned)blocks), dim3(256),
             stream, k, num_rows, stride, slots, cache, num_slots);
  return hipGetLastError();
}

hipError_t launch_quant_q_fold(const uint16_t* q, const float* w_raw, int64_t num_rows,
                               float softmax_scale, float head_norm, uint8_t* q8, float* w_out,
                               float* qs_out, hipStream_t stream) {
  if ((reinterpret_cast<uintptr_t>(q) & 15) == 0) {
    const int64_t blocks = (num_rows + kFoldRows - 1) / kFoldRows;
    IDX_LAUNCH("quant_q_fold16_kernel", (quant_q_fold16_kernel), dim3((unsigned)blocks),
               dim3(256), stream, q, w_raw, num_rows, softmax_scale, head_norm, q8, w_out, qs_out);
    return hipGetLastError();
  }
  const int64_t blocks = (num_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  IDX_LAUNCH("quant_q_fold_kernel", (quant_q_fold_kernel), dim3((unsigned)blocks), dim3(256),
             stream, q, w_raw, num_rows, softmax_scale, head_norm, q8, w_out, qs_out);
  return hipGetLastError();
}

}  // namespace idx

// Device E4M3 quantiser with power-of-two row scales (internal), shared by
// the quantise-and-scatter kernels and the top-k planning kernel, so every
// path writes the same bytes.
//
// encode_e4m3 works on the bf16 bit patterns with integer arithmetic: a row
// scale is a power of two, so x / scale is an exponent shift, and the
// round-to-nearest-even of the E4M3 mantissa is a shift with a sticky test, so
// the result cannot depend on the denormal mode.  The K writes use it.  The
// q-side kernel, which quantises 64 rows per token, uses the hardware
// conversion instead (quant_row_lane8_cvt); the two give the same bytes on
// every finite bf16 value at every row scale (checked exhaustively).
#pragma once

#include "common.hpp"

namespace idx {

// Scale exponent e of a row: the smallest e with max(amax, 1e-4) <= 448 * 2^e.
// `amag` is the bf16 magnitude bit pattern (sign cleared) of the row's amax.
__device__ __forceinline__ int ue8m0_exponent(uint32_t amag) {
  const float a = __uint_as_float(amag << 16);
  if (!(a >= 1e-4f)) return -22;                 // floor: 1e-4 <= 448 * 2^-22
  const int E = (int)(amag >> 7);                // biased exponent (normal here)
  const int m = (int)(amag & 0x7F);
  // a = (1 + m/128) 2^(E-127) and 448 = 1.75 * 2^8
  return (E - 127) - 8 + (m > 96 ? 1 : 0);
}

// E4M3 code of bf16 value x scaled by 2^-e: nearest, ties to even, sign kept,
// saturating at 448 (never reached when e comes from the row's amax).
__device__ __forceinline__ uint32_t encode_e4m3(uint32_t x, int e) {
  const uint32_t sign = (x >> 15) & 1u;
  const uint32_t mag = x & 0x7FFFu;
  if (mag == 0) return sign << 7;
  const int E = (int)(mag >> 7);
  uint32_t M;
  int P;                                          // |x| = M * 2^P
  if (E == 0) { M = mag & 0x7Fu; P = -133; }      // bf16 subnormal
  else { M = 0x80u | (mag & 0x7Fu); P = E - 134; }
  if (E == 0xFF) return (sign << 7) | 0x7Eu;      // inf / nan: saturate (not produced by callers)
  P -= e;
  const int msb = 31 - __clz(M);
  const int j = msb + P;                          // floor(log2 |y|)
  const int qexp = j < -6 ? -9 : j - 3;           // E4M3 spacing in that binade
  const int sh = qexp - P;
  uint32_t N;
  if (sh <= 0) {
    N = M << (-sh);
  } else if (sh >= 10) {
    N = 0;                                        // below half a quantum (M < 2^9)
  } else {
    const uint32_t q = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    N = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  uint32_t code = (j >= -6) ? (uint32_t)((j + 6) * 8) + N : N;
  code = code > 0x7Eu ? 0x7Eu : code;
  return (sign << 7) | code;
}

// One 128-wide row per 32 lanes: each lane owns 4 consecutive values.
// Returns this lane's 4 codes packed little-endian and the row exponent.
__device__ __forceinline__ uint32_t quant_row_lane(uint2 v, int* e_out) {
  const uint32_t x0 = v.x & 0xFFFFu, x1 = v.x >> 16, x2 = v.y & 0xFFFFu, x3 = v.y >> 16;
  uint32_t am = max(max(x0 & 0x7FFFu, x1 & 0x7FFFu), max(x2 & 0x7FFFu, x3 & 0x7FFFu));
  // NaN patterns compare above every finite magnitude; inputs are finite.
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 32));
  const int e = ue8m0_exponent(am);
  *e_out = e;
  return encode_e4m3(x0, e) | (encode_e4m3(x1, e) << 8) | (encode_e4m3(x2, e) << 16) |
         (encode_e4m3(x3, e) << 24);
}

// The same row quantiser with 16 lanes per 128-wide row, 8 consecutive values
// per lane (one 16-byte load).  Returns this lane's 8 codes, little-endian.
__device__ __forceinline__ uint2 quant_row_lane8(uint4 v, int* e_out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 16));
  const int e = ue8m0_exponent(am);
  *e_out = e;
  uint2 c;
  c.x = encode_e4m3(w[0] & 0xFFFFu, e) | (encode_e4m3(w[0] >> 16, e) << 8) |
        (encode_e4m3(w[1] & 0xFFFFu, e) << 16) | (encode_e4m3(w[1] >> 16, e) << 24);
  c.y = encode_e4m3(w[2] & 0xFFFFu, e) | (encode_e4m3(w[2] >> 16, e) << 8) |
        (encode_e4m3(w[3] & 0xFFFFu, e) << 16) | (encode_e4m3(w[3] >> 16, e) << 24);
  return c;
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// quant_row_lane8 with the matrix cores' own conversion: x * 2^-e is exact in
// fp32 (a power-of-two scaling of a bf16 value; the results a flush of fp32
// denormals could touch lie far below half an E4M3 quantum and give a signed
// zero either way), and v_cvt_pk_fp8_f32 rounds it to the nearest E4M3 code,
// ties to even, as encode_e4m3 does.  |x * 2^-e| <= 448, so nothing saturates.
__device__ __forceinline__ uint2 quant_row_lane8_cvt(uint4 v, int* e_out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 16));
  const int e = ue8m0_exponent(am);
  *e_out = e;
  const float s = pow2f(-e);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16) * s;
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * s;
  }
  uint2 c;
  c.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  c.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], (int)c.x, true);
  c.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  c.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], (int)c.y, true);
  return c;
}

// Quantise one K row (32 lanes, row pointer `k`) and store it at `slot` of
// the paged cache; slots outside 0..num_slots-1 are skipped.
__device__ __forceinline__ void quant_write_row(const uint16_t* __restrict__ k, int64_t slot,
                                                uint8_t* __restrict__ cache, int64_t num_slots,
                                                int lane) {
  if (slot < 0 || slot >= num_slots) return;
  const uint2 v = *reinterpret_cast<const uint2*>(k + lane * 4);
  int e;
  const uint32_t codes = quant_row_lane(v, &e);
  const int64_t blk = slot / kBlock, off = slot % kBlock;
  uint8_t* base = cache + blk * kBlockBytes;
  *reinterpret_cast<uint32_t*>(base + off * kHeadDim + lane * 4) = codes;
  if (lane == 0) *reinterpret_cast<float*>(base + kCodeBytes + off * 4) = pow2f(e);
}

}  // namespace idx

// FP8 E4M3FN predictor weights -> bf16 at load time.
//
// The Veda R2VA record (first paragraph) stores the predictor in FP8 and
// dequantises it to BF16 when it is loaded.  E4M3FN is the OCP FP8 format:
// sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals m * 2^-9, no
// infinities, S.1111.111 = NaN.  A power-of-two scale keeps the result exact:
// every E4M3 value times 2^e (|e| <= 24) is a bf16 value, so the conversion is
// done by building the bf16 bit pattern directly (integer work, no rounding).
#include "common.h"

namespace veda {
namespace {

__device__ __forceinline__ uint16_t e4m3_to_bf16_bits(uint32_t b, int32_t e2) {
  const uint32_t sign = (b & 0x80u) << 8;
  const uint32_t ef = (b >> 3) & 0xFu;
  const uint32_t m = b & 0x7u;
  if (ef == 0xFu && m == 0x7u) return (uint16_t)(sign | 0x7FC0u);  // NaN
  if (ef == 0 && m == 0) return (uint16_t)sign;                     // +-0
  int32_t exp2v;      // unbiased exponent of the leading one
  uint32_t mant7;     // 7-bit bf16 mantissa
  if (ef == 0) {
    // subnormal m * 2^-9: normalise the 3-bit mantissa
    const int32_t lead = 31 - __builtin_clz(m);   // 0..2
    exp2v = lead - 9;
    mant7 = ((m << (3 - lead)) & 0x7u) << 4;
  } else {
    exp2v = (int32_t)ef - 7;
    mant7 = m << 4;
  }
  const int32_t be = exp2v + e2 + 127;            // biased bf16 exponent, 1..254 for |e2|<=24
  return (uint16_t)(sign | ((uint32_t)be << 7) | mant7);
}

__global__ __launch_bounds__(256) void dequant_e4m3_kernel(const uint8_t* __restrict__ src,
                                                           uint16_t* __restrict__ dst, int64_t n,
                                                           int32_t e2) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 + 3 < n) {
    // four bytes per thread
    uint32_t w = (uint32_t)src[i0] | ((uint32_t)src[i0 + 1] << 8) | ((uint32_t)src[i0 + 2] << 16) |
                 ((uint32_t)src[i0 + 3] << 24);
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[i0 + t] = e4m3_to_bf16_bits((w >> (8 * t)) & 0xFFu, e2);
  } else {
    for (int64_t i = i0; i < n; ++i) dst[i] = e4m3_to_bf16_bits(src[i], e2);
  }
}

}  // namespace

hipError_t launch_dequant_e4m3(const uint8_t* src, void* dst, int64_t n, int32_t pow2_exp,
                               hipStream_t s) {
  const int64_t per_block = 256 * 4;
  const int64_t blocks = (n + per_block - 1) / per_block;
  hipLaunchKernelGGL(dequant_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src,
                     static_cast<uint16_t*>(dst), n, pow2_exp);
  return hipGetLastError();
}

}  // namespace veda

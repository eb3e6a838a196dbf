// FP8 E4M3FN codec: predictor weights -> bf16 at load time, and bf16 Q / K -> E4M3FN
// codes with a per-tensor power-of-two scale for the FP8 Q.K^T attention path.
//
// The Veda R2VA record (first paragraph) stores the predictor in FP8 and
// dequantises it to BF16 when it is loaded.  E4M3FN is the OCP FP8 format:
// sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals m * 2^-9, no
// infinities, S.1111.111 = NaN.  A power-of-two scale keeps the result exact:
// every E4M3 value times 2^e (|e| <= 24) is a bf16 value, so the conversion is
// done by building the bf16 bit pattern directly (integer work, no rounding).
#include "common.h"

#include <algorithm>

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

// ---- bf16 -> E4M3FN with a per-tensor power-of-two scale
//
// The scale is 2^e with e the smallest integer such that max|x| <= 448 * 2^e (448 is
// the largest E4M3FN value), so x * 2^-e is exact and only the rounding to E4M3FN
// (nearest, ties to even) loses anything; no code saturates.  The rounding is the
// hardware conversion (v_cvt_pk_fp8_f32, OCP E4M3FN on gfx950), which gives the same
// codes as nearest-even rounding spelled out in integer arithmetic for every finite
// bf16 value in range (checked exhaustively at three scales, subnormal codes and ties
// included).  Four launches on one stream: clear the maximum, reduce it, turn it into
// the scale, write the codes.

// Rows (b, n) of a [B, n_tokens, H, d] tensor go to workgroups, the H * d / 8 16-byte
// vectors of a row to threads; f gets each vector's element offset and its 16 bytes.  A
// workgroup takes four of its rows at a time, so that a thread has four loads in flight.
template <typename F>
__device__ __forceinline__ void for_each_vector(const LayerDev& L, int64_t n_tokens, const uint16_t* x, F&& f) {
  const int64_t rows = (int64_t)L.B * n_tokens;
  const int sh = L.d == 128 ? 4 : 3;            // log2(d / 8)
  const int per_row = L.H << sh;
  const int64_t stride = gridDim.x;
  for (int64_t r0 = blockIdx.x; r0 < rows; r0 += 4 * stride) {
    int64_t base[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t r = r0 + u * stride;
      ok[u] = r < rows;
      const int64_t b = (ok[u] ? r : r0) / n_tokens;
      base[u] = b * L.sb + ((ok[u] ? r : r0) - b * n_tokens) * L.sn;
    }
    for (int j = threadIdx.x; j < per_row; j += blockDim.x) {
      const int64_t col = (int64_t)(j >> sh) * L.sh + 8 * (j & ((1 << sh) - 1));
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = ok[u] ? *reinterpret_cast<const uint4*>(x + base[u] + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ok[u]) f(base[u] + col, w[u]);
    }
  }
}

__global__ void fp8_clear_kernel(uint32_t* word) { *word = 0u; }

// largest |x| as the bit pattern of a non-negative float (integer order = value order)
__global__ __launch_bounds__(256) void fp8_amax_kernel(LayerDev L, int64_t n_tokens,
                                                        const uint16_t* __restrict__ x,
                                                        uint32_t* __restrict__ word) {
  uint32_t m = 0;
  for_each_vector(L, n_tokens, x, [&](int64_t, const uint4& w) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      m = max(m, a[t] & 0x7FFFu);
      m = max(m, (a[t] >> 16) & 0x7FFFu);
    }
  });
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(part[0], part[1]), max(part[2], part[3]));
    if (m) atomicMax(word, m << 16);
  }
}

// the word becomes the float scale 2^e
__global__ void fp8_scale_kernel(uint32_t* word) {
  const float amax = __uint_as_float(*word);
  int e = 0;
  if (amax > 0.f) {
    int ex;
    const float f = frexpf(amax, &ex);          // amax = f * 2^ex, f in [0.5, 1)
    // 448 * 2^e = 1.75 * 2^(e + 8) >= amax = 2f * 2^(ex - 1)
    e = f <= 0.875f ? ex - 9 : ex - 8;
  }
  *reinterpret_cast<float*>(word) = ldexpf(1.0f, e);
}

__global__ __launch_bounds__(256) void fp8_quantize_kernel(LayerDev L, int64_t n_tokens,
                                                            const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ x8,
                                                            const float* __restrict__ scale) {
  int ex;
  frexpf(scale[0], &ex);
  const int e = ex - 1;                          // scale = 2^e
  for_each_vector(L, n_tokens, x, [&](int64_t off, const uint4& w) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
    float f[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f[2 * t] = ldexpf(__uint_as_float(a[t] << 16), -e);
      f[2 * t + 1] = ldexpf(__uint_as_float(a[t] & 0xFFFF0000u), -e);
    }
    int c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], c0, true);
    int c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], c1, true);
    *reinterpret_cast<uint2*>(x8 + off) = make_uint2((uint32_t)c0, (uint32_t)c1);
  });
}

// V for the FP8 attention's second product, d-major in blocks of 64 tokens: block
// (b, h, g) is d rows of 64 bytes, row c holding the codes of V[b, 64 g + t, h, c] for
// t = 0..63 (zeros past the last token), its four 16-byte chunks XOR-swizzled by
// (c >> 1) & 3 so that the kernel's operand reads (eight consecutive rows, one chunk
// each) hit distinct LDS banks.  One workgroup quantises one block through LDS.
template <int D>
__global__ __launch_bounds__(256) void fp8_quantize_vt_kernel(LayerDev L, int64_t n_tokens, int64_t n_blocks,
                                                               const uint16_t* __restrict__ x,
                                                               uint8_t* __restrict__ vt,
                                                               const float* __restrict__ scale) {
  __shared__ uint8_t tile[64][D + 4];           // token-major codes of the block
  int ex;
  frexpf(scale[0], &ex);
  const int e = ex - 1;                          // scale = 2^e
  const int64_t blk = blockIdx.x;
  const int64_t g = blk % n_blocks;
  const int64_t bh = blk / n_blocks;
  const int64_t h = bh % L.H, b = bh / L.H;
  constexpr int VPR = D / 8;                     // 8-element vectors per token row
  for (int u = threadIdx.x; u < 64 * VPR; u += 256) {
    const int t = u / VPR, c8 = u % VPR;
    const int64_t n = 64 * g + t;
    uint32_t c[2] = {0u, 0u};
    if (n < n_tokens) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + b * L.sb + n * L.sn + h * L.sh + 8 * c8);
      const uint32_t a[4] = {w.x, w.y, w.z, w.w};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = ldexpf(__uint_as_float(a[i] << 16), -e);
        f[2 * i + 1] = ldexpf(__uint_as_float(a[i] & 0xFFFF0000u), -e);
      }
      int c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], c0, true);
      int c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
      c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], c1, true);
      c[0] = (uint32_t)c0;
      c[1] = (uint32_t)c1;
    }
    *reinterpret_cast<uint32_t*>(&tile[t][8 * c8]) = c[0];
    *reinterpret_cast<uint32_t*>(&tile[t][8 * c8 + 4]) = c[1];
  }
  __syncthreads();
  uint8_t* const dst = vt + blk * (int64_t)(D * 64);
  for (int u = threadIdx.x; u < D * 4; u += 256) {
    const int c = u >> 2, pc = u & 3;
    const int lc = pc ^ ((c >> 1) & 3);          // logical chunk: tokens 16 lc .. 16 lc + 15
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t0 = 16 * lc + 4 * q;
      w[q] = (uint32_t)tile[t0][c] | ((uint32_t)tile[t0 + 1][c] << 8) | ((uint32_t)tile[t0 + 2][c] << 16) |
             ((uint32_t)tile[t0 + 3][c] << 24);
    }
    *reinterpret_cast<uint4*>(dst + c * 64 + pc * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_quantize_fp8_vt(const LayerDev& L, int64_t n_tokens, const void* v, uint8_t* vt,
                                  float* scale, hipStream_t s) {
  const int64_t amax_blocks = std::min<int64_t>((int64_t)L.B * n_tokens, 8192);
  const int64_t n_blocks = (n_tokens + 63) / 64;
  const int64_t grid = (int64_t)L.B * L.H * n_blocks;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  uint32_t* word = reinterpret_cast<uint32_t*>(scale);
  auto xx = static_cast<const uint16_t*>(v);
  hipLaunchKernelGGL(fp8_clear_kernel, dim3(1), dim3(1), 0, s, word);
  hipLaunchKernelGGL(fp8_amax_kernel, dim3((unsigned)amax_blocks), dim3(256), 0, s, L, n_tokens, xx, word);
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(1), dim3(1), 0, s, word);
  if (L.d == 128)
    hipLaunchKernelGGL((fp8_quantize_vt_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, L, n_tokens, n_blocks,
                       xx, vt, scale);
  else
    hipLaunchKernelGGL((fp8_quantize_vt_kernel<64>), dim3((unsigned)grid), dim3(256), 0, s, L, n_tokens, n_blocks,
                       xx, vt, scale);
  return hipGetLastError();
}

hipError_t launch_dequant_e4m3(const uint8_t* src, void* dst, int64_t n, int32_t pow2_exp,
                               hipStream_t s) {
  const int64_t per_block = 256 * 4;
  const int64_t blocks = (n + per_block - 1) / per_block;
  hipLaunchKernelGGL(dequant_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src,
                     static_cast<uint16_t*>(dst), n, pow2_exp);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const LayerDev& L, int64_t n_tokens, const void* x, uint8_t* x8,
                                float* scale, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((int64_t)L.B * n_tokens, 8192);
  uint32_t* word = reinterpret_cast<uint32_t*>(scale);
  auto xx = static_cast<const uint16_t*>(x);
  hipLaunchKernelGGL(fp8_clear_kernel, dim3(1), dim3(1), 0, s, word);
  hipLaunchKernelGGL(fp8_amax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, L, n_tokens, xx, word);
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(1), dim3(1), 0, s, word);
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, L, n_tokens, xx, x8,
                     scale);
  return hipGetLastError();
}

}  // namespace veda

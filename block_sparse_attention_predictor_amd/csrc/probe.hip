// Measurement aid (libveda_probe.so, declared in include/veda_probe.h): the bf16
// matrix-core rate an MFMA-only loop reaches on this device, the reference against
// which a benchmark also reports the attention kernel's MFMA use (besides the
// 2.5 PFLOP/s specification).  Not part of the method's library.
#include "../../include/veda_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every wave runs iters x 16 products of v_mfma_f32_32x32x16_bf16 on four
// independent accumulators (32768 flops each); the sums are stored so that nothing
// is optimised away.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)(i - (int)(threadIdx.x & 7)));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int veda_probe_mfma_peak(float* out, int32_t iters, int32_t workgroups, void* stream) {
  if (!out || iters < 1 || workgroups < 1) return -1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

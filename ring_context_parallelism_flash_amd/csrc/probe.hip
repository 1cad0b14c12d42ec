// Matrix-core throughput probe: confirms on the device the dense bf16 rate
// per compute unit per clock that the attention kernels' roofline is priced
// against. Every wave issues register-fed v_mfma_f32_32x32x16_bf16 on four
// independent accumulators (no operand loads, no dependency stalls) and
// records the shader-clock counter (s_memtime) and the constant 100 MHz
// reference counter (s_memrealtime) at its start and end. One workgroup of 8
// waves runs on a compute unit at a time (the dynamic LDS request leaves room
// for one), so each SIMD holds two waves and its matrix pipe never waits for
// an issue slot; the host takes a workgroup's span from its earliest start
// to its latest end, so waves that start late do not inflate the rate.
#include <hip/hip_runtime.h>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float floatx16_p __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kProbeThreads, 1) void mfma_bf16_probe(int32_t iters,
                                                                     int64_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  bf16x8_p a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (lane + j));
    b[j] = (__bf16)(0.002f * (lane - j));
  }
  floatx16_p acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  const int64_t c0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[kProbeWords * wave + 0] = c0;
    out[kProbeWords * wave + 2] = r0;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[t][i];
  const int64_t c1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[kProbeWords * wave + 1] = c1;
    out[kProbeWords * wave + 3] = r1;
  }
  if (lane == 1) out[kProbeWords * wave + 4] = (int64_t)(sum != sum);  // keeps the products live
}

}  // namespace

hipError_t launch_mfma_probe(int32_t workgroups, int32_t iters, int64_t* out, hipStream_t s) {
  const void* fn = (const void*)mfma_bf16_probe;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kProbeLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mfma_bf16_probe, dim3((unsigned)workgroups), dim3(kProbeThreads),
                     kProbeLdsBytes, s, iters, out);
  return hipGetLastError();
}

}  // namespace ra

// MFMA-only throughput probe: every CU runs four waves that issue nothing but
// independent v_mfma_f32_32x32x16_bf16 (eight accumulator chains per wave), with
// operands that either stay constant or change from one MFMA to the next
// (pseudo-random bf16 values). It measures the bf16 MFMA rate and the shader
// clock (s_memtime ticks over s_memrealtime ticks) the part sustains with no
// memory traffic at all: the ceiling any bf16 GEMM on this part runs under.
#include "ptg_device.hpp"

namespace ptg {

__device__ __forceinline__ float probe_value(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return (float)((int32_t)(x & 0xFFFFu) - 32768) * (1.0f / 32768.0f);
}

template <bool VARY>
__global__ __launch_bounds__(256, 1) void ptg_mfma_probe_kernel(int32_t iters, float *sink, uint64_t *ticks) {
  bf16x8 a[4], b[4];
  for (int r = 0; r < 4; ++r)
    for (int i = 0; i < 8; ++i) {
      const uint32_t id = threadIdx.x * 64u + (uint32_t)(r * 8 + i);
      a[r][i] = (__bf16)(VARY ? probe_value(id + blockIdx.x * 7919u) : 0.01f);
      b[r][i] = (__bf16)(VARY ? probe_value(id + 100003u + blockIdx.x * 104729u) : 0.02f);
    }
  const uint64_t t0 = clock_core(), r0 = clock_wall();
  f32x16 acc[8];
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 1) & 3], acc[j], 0, 0, 0);
  }
  float s = 0.0f;
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[blockIdx.x * 256u + threadIdx.x] = s;  // keeps the MFMAs alive
  const uint64_t t1 = clock_core(), r1 = clock_wall();
  if (threadIdx.x == 0) {
    ticks[blockIdx.x * 2u] = t1 - t0;
    ticks[blockIdx.x * 2u + 1u] = r1 - r0;
  }
}

hipError_t launch_mfma_probe(int grid, int32_t iters, bool vary, float *sink, uint64_t *ticks, hipStream_t s) {
  if (vary)
    hipLaunchKernelGGL(ptg_mfma_probe_kernel<true>, dim3(grid), dim3(256), 0, s, iters, sink, ticks);
  else
    hipLaunchKernelGGL(ptg_mfma_probe_kernel<false>, dim3(grid), dim3(256), 0, s, iters, sink, ticks);
  return hipGetLastError();
}

}  // namespace ptg

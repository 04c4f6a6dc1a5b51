// MFMA-only throughput probe: every CU runs four waves that issue nothing but
// independent bf16 MFMAs into accumulators that stay in place (assembly
// statements, so the compiler cannot rotate accumulators through copies), with
// operands that either stay constant or differ from one MFMA to the next
// (pseudo-random bf16 values in four register sets). One round per wave is
// eight v_mfma_f32_32x32x16_bf16 or sixteen v_mfma_f32_16x16x32_bf16: the same
// 262144 flop either way. It measures the bf16 MFMA rate and the shader clock
// (s_memtime ticks over s_memrealtime ticks) the part sustains with no memory
// traffic at all: the ceiling a bf16 GEMM built on that instruction runs under.
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

template <bool VARY, int MB>
__global__ __launch_bounds__(256, 1) void ptg_mfma_probe_kernel(int32_t iters, float *sink, uint64_t *ticks) {
  // MB = 32: eight 32x32 accumulators of 16 floats; MB = 16: sixteen 16x16 accumulators of 4 floats
  constexpr int NACC = MB == 32 ? 8 : 16;
  constexpr int ACCN = MB == 32 ? 16 : 4;
  typedef float accv __attribute__((ext_vector_type(ACCN)));
  bf16x8 a[4], b[4];
  for (int r = 0; r < 4; ++r)
    for (int i = 0; i < 8; ++i) {
      const uint32_t id = threadIdx.x * 64u + (uint32_t)(r * 8 + i);
      a[r][i] = (__bf16)(VARY ? probe_value(id + blockIdx.x * 7919u) : 0.01f);
      b[r][i] = (__bf16)(VARY ? probe_value(id + 100003u + blockIdx.x * 104729u) : 0.02f);
    }
  const uint64_t t0 = clock_core(), r0 = clock_wall();
  accv acc[NACC];
  for (int j = 0; j < NACC; ++j)
    for (int e = 0; e < ACCN; ++e) acc[j][e] = 0.0f;
  // the zeroed accumulators in their registers, then wait states before the first MFMA reads them
#pragma unroll
  for (int j = 0; j < NACC; ++j) asm volatile("" : "+a"(acc[j]));
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
      if constexpr (MB == 32)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a[j & 3]), "v"(b[(j >> 1) & 3]));
      else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a[j & 3]), "v"(b[(j >> 2) & 3]));
    }
  }
  // wait states after the last MFMA before its result is read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < NACC; ++j) asm volatile("" : "+a"(acc[j]));
  float s = 0.0f;
  for (int j = 0; j < NACC; ++j)
    for (int e = 0; e < ACCN; ++e) s += acc[j][e];
  sink[blockIdx.x * 256u + threadIdx.x] = s;  // keeps the MFMAs alive
  const uint64_t t1 = clock_core(), r1 = clock_wall();
  if (threadIdx.x == 0) {
    ticks[blockIdx.x * 2u] = t1 - t0;
    ticks[blockIdx.x * 2u + 1u] = r1 - r0;
  }
}

hipError_t launch_mfma_probe(int grid, int32_t iters, bool vary, int mfma_block, float *sink, uint64_t *ticks,
                             hipStream_t s) {
  if (mfma_block == 32) {
    if (vary)
      hipLaunchKernelGGL((ptg_mfma_probe_kernel<true, 32>), dim3(grid), dim3(256), 0, s, iters, sink, ticks);
    else
      hipLaunchKernelGGL((ptg_mfma_probe_kernel<false, 32>), dim3(grid), dim3(256), 0, s, iters, sink, ticks);
  } else if (mfma_block == 16) {
    if (vary)
      hipLaunchKernelGGL((ptg_mfma_probe_kernel<true, 16>), dim3(grid), dim3(256), 0, s, iters, sink, ticks);
    else
      hipLaunchKernelGGL((ptg_mfma_probe_kernel<false, 16>), dim3(grid), dim3(256), 0, s, iters, sink, ticks);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ptg

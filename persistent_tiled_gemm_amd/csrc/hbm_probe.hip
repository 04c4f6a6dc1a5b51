// Memory-only probe (a fact about the part, no page behind it): the bandwidth
// a plain streaming kernel reaches, as the practical ceiling the HBM-bound GEMM
// shapes are compared with beside the 8 TB/s of the data sheet. Two kernels
// over buffers twice the last-level cache: a read-only pass (16-byte
// non-temporal loads per lane, grid-stride, summed so the loads stay live)
// and a copy (16-byte non-temporal load and store per lane).
#include "ptg_device.hpp"

namespace ptg {

__global__ __launch_bounds__(256) void ptg_hbm_read_kernel(const f32x4 *src, size_t n, float *sink) {
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const f32x4 a = __builtin_nontemporal_load(src + i);
    const f32x4 b = __builtin_nontemporal_load(src + i + stride);
    const f32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const f32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc += (a + b) + (c + d);
  }
  for (; i < n; i += stride) acc += __builtin_nontemporal_load(src + i);
  const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  // the buffer holds zeros, so this never stores; it keeps the loads from being removed
  if (s != 0.0f) sink[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void ptg_hbm_copy_kernel(const f32x4 *src, f32x4 *dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_hbm_probe(int kind, int grid, const void *src, void *dst, size_t bytes, float *sink,
                            hipStream_t s) {
  const size_t n = bytes / sizeof(f32x4);
  if (kind == 0)
    hipLaunchKernelGGL(ptg_hbm_read_kernel, dim3(grid), dim3(256), 0, s, static_cast<const f32x4 *>(src), n, sink);
  else
    hipLaunchKernelGGL(ptg_hbm_copy_kernel, dim3(grid), dim3(256), 0, s, static_cast<const f32x4 *>(src),
                       static_cast<f32x4 *>(dst), n);
  return hipGetLastError();
}

}  // namespace ptg

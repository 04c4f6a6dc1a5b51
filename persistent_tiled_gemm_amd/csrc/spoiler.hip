// Spoiler: occupy compute units for a fixed time, to create the "part of the
// machine is busy with another kernel" condition under which a fixed task
// sequence tails (blog post "CUTLASS Cluster Launch Control dynamic persistent
// kernel", section "why a fixed task sequence tails").
//
// Each workgroup is one wave that asks for all of a CU's LDS (dynamic shared
// memory), so no other workgroup can share its CU while it runs. It records
// its start time and placement, announces itself on a host-visible counter and
// spins on the constant-rate clock until its time is up. The wait is bounded by
// construction: it ends when the clock passes the deadline.
#include "ptg_device.hpp"

namespace ptg {

__global__ __launch_bounds__(64, 1) void ptg_spoiler_kernel(uint64_t spin_ticks, uint32_t *resident,
                                                            uint64_t *log) {
  extern __shared__ unsigned char spoiler_lds[];
  const uint64_t r0 = clock_wall();
  if (threadIdx.x == 0) {
    spoiler_lds[0] = 1;  // the LDS reservation is what pins the CU; touch it once
    if (resident) __hip_atomic_fetch_add(resident, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  const uint64_t deadline = r0 + spin_ticks;
  uint64_t now = r0;
  while (now < deadline) {
    __builtin_amdgcn_s_sleep(32);
    now = clock_wall();
  }
  if (threadIdx.x == 0 && log) {
    uint64_t *o = log + 4 * (size_t)blockIdx.x;
    o[0] = r0;
    o[1] = now;
    o[2] = read_hw_id();
    o[3] = read_xcc_id();
  }
}

hipError_t launch_spoiler(int n_wgs, uint64_t spin_ticks, uint32_t *resident, uint64_t *log, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int lds = 0;
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ptg_spoiler_kernel, dim3(n_wgs), dim3(64), lds, stream, spin_ticks, resident, log);
  return hipGetLastError();
}

}  // namespace ptg

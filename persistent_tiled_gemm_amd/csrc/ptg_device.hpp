// Device-side building blocks of the persistent tiled GEMM (gfx950 only):
// operand types, buffer resources with out-of-range masking, timers and
// hardware ids, the tile raster and the claim-ring record.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ptg_internal.hpp"

namespace ptg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Buffer resource over a base pointer. Offsets at or above kBufRecords read as
// zero (hardware range check), which is how edge rows/columns and the K tail
// are masked: a lane whose chunk lies outside the matrix gets kBufOob.
static constexpr uint32_t kBufRecords = 0x40000000u;
static constexpr uint32_t kBufOob = 0x40000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
  // word 3 = 0x00020000: raw (untyped) 32-bit data format for gfx9-family buffers
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)kBufRecords, 0x00020000);
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

// The same resource as four SGPR words, for inline assembly (the base must be
// wave-uniform; readfirstlane makes that explicit to the compiler).
__device__ __forceinline__ i32x4 make_rsrc_words(const void *base) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));  // stride 0
  r[2] = (int)kBufRecords;
  r[3] = 0x00020000;
  return r;
}

// The same with a record count of zero when !live: every load through it then
// reads zeros (a whole k-step masked with one scalar select, no branch).
__device__ __forceinline__ i32x4 make_rsrc_words(const void *base, bool live) {
  i32x4 r = make_rsrc_words(base);
  r[2] = live ? (int)kBufRecords : 0;
  return r;
}

// 16-byte accesses for data that a workgroup on another XCD reads later in
// the same run (the split tail's partial sums). The sc1 cache-policy bit (bit
// 4 of the buffer builtins' policy operand on gfx950) is what the compiler
// puts on agent-scope atomic loads and stores: the store writes through this
// XCD's L2 and the load fetches past the reader's. With every access to that
// data made this way, waiting for the stores (vmcnt(0)) orders them before a
// later atomic, so no fence is needed; a device-scope fence would write back
// and invalidate the whole L2 of the XCD, which costs the other workgroups on
// it their cached operands.
static constexpr int kPolicyAgent = 16;
__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t r, uint32_t offset, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)offset, 0, kPolicyAgent);
}
__device__ __forceinline__ f32x4 load16_agent(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, kPolicyAgent));
}

template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T *>(((uint64_t)hi << 32) | lo);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p);
}

// 16 bytes per lane from global memory straight into LDS at lds_base + lane*16
// (lds_base is wave-uniform; the instruction takes it from M0, which the
// statement names as an input so that the compiler itself sets M0 and knows the
// statement reads it). Issued as inline assembly so the compiler does not add a
// conservative wait before every later LDS read: the kernel waits for these
// loads itself (vmcnt) before the barrier that publishes the stage.
__device__ __forceinline__ void load16_to_lds(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile("buffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voffset), "{m0}"(lds_base), "s"(rsrc)
               : "memory");
}

__device__ __forceinline__ void wait_lds_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Execution barrier for the workgroup without the full-memory fence of
// __syncthreads (the direct-to-LDS loads are waited for explicitly).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint64_t clock_core() { return __builtin_amdgcn_s_memtime(); }
__device__ __forceinline__ uint64_t clock_wall() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t read_hw_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
  return v;
}
__device__ __forceinline__ uint32_t read_xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}

__device__ __forceinline__ uint32_t wave_uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Tile id -> (m_t, n_t) inside one problem. Row-major, or grouped-M: groups of
// `group` tile rows, column-major inside a group (so consecutive ids share B
// column panels and a few A row panels).
__device__ __forceinline__ void decode_tile(int32_t t, int32_t tiles_m, int32_t tiles_n, int32_t group,
                                            int32_t &m_t, int32_t &n_t) {
  if (group <= 1) {
    m_t = t / tiles_n;
    n_t = t - m_t * tiles_n;
    return;
  }
  const int32_t per_group = group * tiles_n;
  const int32_t g = t / per_group;
  const int32_t first_m = g * group;
  int32_t gm = tiles_m - first_m;
  gm = gm < group ? gm : group;
  const int32_t r = t - g * per_group;
  m_t = first_m + r % gm;
  n_t = r / gm;
}

// Which entry of a grouped launch's table owns work unit u: the last entry
// whose unit_start is <= u. unit_start ascends (the table is in claim order;
// an entry with no units shares its unit_start with the next one), so the
// entries with unit_start <= u are a prefix of the table and the answer is
// their count less one. Called by whole waves with a wave-uniform u: lane l
// tests entries l, l + 64, ..., four loads at a time. The loads are
// independent, so a table of up to 256 entries costs one load round trip (a
// binary search costs log2 G dependent ones: on 64 problems, about 5 us of a
// 600 us launch).
__device__ __forceinline__ int32_t find_problem(const KernelProblem *probs, int32_t G, int32_t u) {
  const int32_t lane = (int32_t)(threadIdx.x & 63u);
  int32_t count = 0;
  for (int32_t base = 0; base < G; base += 256) {
    int32_t us[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t i = base + 64 * q + lane;
      us[q] = probs[i < G ? i : 0].unit_start;  // lanes past the end reload entry 0
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) count += __popcll(__ballot(base + 64 * q + lane < G && us[q] <= u));
  }
  return count - 1;
}

}  // namespace ptg

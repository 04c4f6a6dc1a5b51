// Persistent tiled bf16 GEMM for gfx950: C (fp32) = A (bf16, M x K) . B (bf16, K x N).
//
// One workgroup = a 2 x 2 grid of wave64s. 256 x 256 tiles: one workgroup per
// CU, each wave owns 128 x 128 of the tile as 8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16 (one wave per SIMD). 128 x 128 tiles: two
// workgroups per CU, each wave owns 64 x 64 as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16. Accumulation is fp32 throughout. Operand tiles move
// global -> LDS with buffer_load_dwordx4 ... lds (16 bytes per lane, no VGPR
// round trip) into a ring of four 32-deep LDS stages, each load two to three
// k-steps ahead of its first reader.
//
// LDS layouts: the four B stages first, then the four A stages (so that reads
// of a stage known at compile time need no address arithmetic in the loop);
// 16-byte chunks, XOR-swizzled so fragment reads are bank-conflict free:
//   A stage: BM rows x 32 k, 64 B per row; logical chunk c of row r sits in slot
//            c ^ ((r >> 1) & 3) (16 x 16 blocks) or c ^ ((r >> 2) & 3) (32 x 32).
//            A fragments are read with ds_read_b128 (8 consecutive k of one row
//            per lane).
//   B stage: 32 k rows x BN n; logical chunk c of row k sits in slot
//            c ^ s(k), s(k) = (10 (k & 1) + 4 ((k >> 1) & 1)) ^ 2 ((k >> 3) & 1).
//            B fragments need 8 consecutive k of one column per lane;
//            ds_read_b64_tr_b16 delivers them from the row-major (n-contiguous)
//            tile: in each 16-lane group, lane L reads 4 n values of row L/4 and
//            lane i receives column i of the 4 x 16 block.
// The MFMA is issued with the B fragment as its first operand, so each group of
// four accumulators of a lane holds four consecutive n of one row m, which the
// epilogue writes as one 16-byte store.
//
// Work units. The schedulers hand out work units; a unit is one work item, or
// with claim groups g consecutive items that one worker runs back to back. An
// item is a whole tile, or with a split tail one K-chunk of a tile of the
// partial last wave: a chunk stores its fp32 partial tile to plan scratch and
// the workgroup that completes the tile's last chunk adds the partials in chunk
// order and writes C (no workgroup ever waits for another).
//
// Scheduling: see the header comment of ptg_gemm.h. The work loop is the
// persistent worker loop of the blog post "CUTLASS Cluster Launch Control
// dynamic persistent kernel" (section "cancelling the launch, receiving the
// work coordinate": compute the tile, fetch the next coordinate, stop on
// failure); the claim-ahead and its LDS ring of response records follow its
// section "following the CUTLASS source" (one elected producer thread, a
// depth-3 response pipeline, a throttle on how far ahead claims run, consumers
// check the success flag before the coordinate).
#include <type_traits>

#include "ptg_device.hpp"

namespace ptg {

// Tile shape, wave grid and MFMA shape. A workgroup has WAVES_M x WAVES_N
// wave64s; each wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of the output
// tile, made of MB x MB MFMA blocks: MB = 32 uses v_mfma_f32_32x32x16_bf16 (two
// MFMAs per 32-deep stage), MB = 16 uses v_mfma_f32_16x16x32_bf16 (one).
template <int BM, int BN, int WAVES_M, int WAVES_N, int MB_>
struct Cfg {
  static constexpr int BM_ = BM, BN_ = BN, WAVES_N_ = WAVES_N;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BK = 32, NSTAGE = 4;          // k per stage, LDS stages
  static constexpr int MB = MB_, KS = 512 / MB_;     // MFMA block edge, k per MFMA
  static constexpr int ACC_N = MB * MB / 64;         // accumulator floats per lane per block
  static constexpr int QUADS = ACC_N / 4;            // 16-byte groups of them
  static constexpr int A_ROW = BK * 2;              // bytes per row of the A stage
  static constexpr int A_ROW_CHUNKS = BK / 8;
  static constexpr int A_RPL = 1024 / A_ROW;         // A rows one wave-load (64 x 16 B) covers
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // wave tile
  static constexpr int MI = WM / MB, NI = WN / MB;            // MFMA blocks per wave
  static constexpr int A_LOADS = BM * (BK / 8) / THREADS;     // 16-byte loads per thread per stage
  static constexpr int B_LOADS = BK * (BN / 8) / THREADS;
  static constexpr int A_STAGE = BM * BK * 2;       // bytes
  static constexpr int B_STAGE = BK * BN * 2;
  static constexpr int B_ROW = BN * 2;              // bytes per k row of the B stage
  static constexpr int B_ROW_CHUNKS = BN / 8;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS = NSTAGE * STAGE;
  // LDS placement: the four B stages first, then the four A stages, so that
  // every fragment read of a stage known at compile time is a per-lane base
  // plus an offset that fits the 16-bit offset field of ds_read (the A base
  // carries the B region's size)
  static constexpr int B_REGION = NSTAGE * B_STAGE;
  static constexpr int a_off(int s) { return B_REGION + s * A_STAGE; }
  static constexpr int b_off(int s) { return s * B_STAGE; }
  static_assert(A_LOADS * THREADS == BM * (BK / 8) && B_LOADS * THREADS == BK * (BN / 8), "load split");
  static_assert(WM % MB == 0 && WN % MB == 0 && (MB == 16 || MB == 32), "wave tile");
};

// The wave grid used for each tile edge: 128 -> 2 x 2 waves of 64 x 64 in
// 32 x 32 blocks (two workgroups per CU, so two waves share each SIMD); 256 ->
// 2 x 2 waves of 128 x 128 in 16 x 16 blocks (one wave per SIMD, 256
// accumulator registers each). The large wave tile reads two thirds of the LDS
// bytes per flop that 128 x 64 wave tiles need, and the part is power-bound,
// so fewer LDS bytes buy clock.
template <int EDGE> struct TileCfg;
template <> struct TileCfg<128> { using type = Cfg<128, 128, 2, 2, 32>; };
template <> struct TileCfg<256> { using type = Cfg<256, 256, 2, 2, 16>; };

// A: the slot XOR for row r depends on the fragment read pattern. Measured with
// the LDS bank-conflict counter on gfx950 (ds_read_b128, 64 B rows): for 32 x 32
// blocks (32 rows x one chunk per half-wave) (r >> 2) & 3 is conflict-free and
// (r >> 1) & 3 is two-way; for 16 x 16 blocks (16 rows x four chunks) it is the
// other way round, and no XOR at all is two-way.
template <int MB>
__device__ __forceinline__ uint32_t swz_a(uint32_t row) { return MB == 32 ? (row >> 2) & 3u : (row >> 1) & 3u; }
__device__ __forceinline__ uint32_t swz_b(uint32_t k) {
  return (10u * (k & 1u) + 4u * ((k >> 1) & 1u)) ^ (2u * ((k >> 3) & 1u));
}

// One record of the claim ring: the answer to one claim. `valid` is the success
// predicate; `tile` is meaningful only when valid. `seq` is the worker's tile
// ordinal the record answers (checked by the consumers).
struct RingRec {
  uint32_t tile, valid, seq, pad;
};

static constexpr int kRingDepth = 3;  // LDS slots; a run uses args.ring_depth (2 or 3) of them

// Record a device-side failure: in this run's control block (bit set of the
// run) and in the plan's status word, which only the host clears, so a failure
// of any run stays visible until the host has read it.
__device__ __forceinline__ void flag_error(const KernelArgs &a, uint32_t bit) {
  __hip_atomic_fetch_or(&a.ctrl->error, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_or(a.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rotation of a unit's K order: the physical k-step its logical step kb + i
// reads is kb + ((i + rot) mod nsteps) (see the K order at the item set-up).
// `item` is the key the phase follows: the item id, or a grouped run's problem.
__device__ __forceinline__ int32_t k_rotation_of(const KernelArgs &a, uint32_t item, int32_t nsteps) {
  if (a.k_rotation == 0 || nsteps <= 1) return 0;
  uint32_t rot;
  if (a.k_rotation == 1 || a.k_rotation == 2) {
    // one phase per XCD region (item id mod 8; a plain launch sends item i to
    // XCD i mod 8): the workgroups of one XCD, which share operand panels
    // through its L2, keep walking K together. Or two phases per region (item
    // id mod 16), half the range apart.
    const uint32_t phases = a.k_rotation == 1 ? (uint32_t)kXcdRegions : 2u * kXcdRegions;
    rot = (item % phases) * (uint32_t)nsteps / phases;
  } else {
    // a phase per unit (multiplicative hash of the item id)
    rot = ((item * 2654435761u) >> 16) % (uint32_t)nsteps;
  }
  return (int32_t)wave_uniform(rot);
}

// Thread 0 of every workgroup, once, after its last use of the run's scheduler
// state, in runs that clean up after themselves (self_clean: launches captured
// into a graph, which replay on one state set): count the workgroup out; the
// last one of the grid resets the claim counters, the gate and the count
// itself, so the next replay starts from zero without a host-side reset. Other
// runs skip it: the plan's next run clears their set before it is used again
// (the count's two dependent atomics at the end of a launch cost 2-4 us).
// The count has two levels: a workgroup counts into its group (blockIdx mod
// kExitGroups, one cache line per group), and the workgroup that completes a
// group counts the group into exit_count; the one that completes the last
// group resets everything. (With one counter, the late launch slots of a
// dynamic run, thousands for small tiles, all hit one address at the end:
// 8192^3 with 128 x 128 tiles lost ~125 us to it.)
// Relaxed order is enough: a workgroup's claims are returning atomics whose
// answers it has waited for, so they are performed before its count goes out;
// the resetting workgroup resets only after its own counts have come back; and
// the next launch that reads this state starts after this kernel has ended,
// which orders everything before it. (An acquire-release count writes back and
// invalidates the XCD's whole L2 in every exiting workgroup, which the workers
// still running on that XCD then pay for: 8192^3 static 750 -> 741 us and
// dynamic 773 -> 755 us without it.)
__device__ __forceinline__ void leave_run(const KernelArgs &a) {
  const uint32_t g = blockIdx.x % (uint32_t)kExitGroups;
  const uint32_t in_group = (gridDim.x - g + (uint32_t)kExitGroups - 1u) / (uint32_t)kExitGroups;
  const uint32_t groups = min(gridDim.x, (uint32_t)kExitGroups);
  const uint32_t done =
      __hip_atomic_fetch_add(&a.ctrl->exit_group[g * kExitStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (done + 1u != in_group) return;
  const uint32_t groups_done = __hip_atomic_fetch_add(&a.ctrl->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (groups_done + 1u == groups) {
    __hip_atomic_store(&a.ctrl->counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.ctrl->gate, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.ctrl->error, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int x = 0; x < kXcdRegions; ++x)
      __hip_atomic_store(&a.ctrl->xcd_counter[(x) * kXcdStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int x = 0; x < kExitGroups; ++x)
      __hip_atomic_store(&a.ctrl->exit_group[x * kExitStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.ctrl->exit_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Ask the scheduler for an alternation of one MFMA and one LDS read in the
// current scheduling region (then the remaining MFMAs or reads).
template <int READS, int MFMAS>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < MFMAS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
    if (i < READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  if constexpr (READS > MFMAS) __builtin_amdgcn_sched_group_barrier(0x100, READS - MFMAS, 0);
}

// One claim. Single-counter policy: the next value of the device-wide counter
// (plus the failure-forcing base); any value >= T is a failure. XCD-partitioned
// policies: region x (tiles 8i + x, or the x-th of eight consecutive runs of
// ids; see region_unit) is handed out by counter x; a worker claims
// from its own XCD's region first (the tiles its XCD's L2 already holds
// operands for) and, once that is exhausted, steals from another region. Each
// counter returns each index once, so every tile still has exactly one owner;
// the claim fails (returns T) only when every region is exhausted.
//
// A claim is split in two. claim_issue sends the first atomic (the global
// counter, or the counter of the worker's current region: its own XCD's to
// begin with) from lane 0 and returns its raw answer in lane 0's register,
// valid once the wave's memory operations have drained (vmcnt 0); the round
// trip hides under the MFMAs of the current tile. claim_resolve, called by a whole wave (all lanes active) once
// the answer is needed, broadcasts it and turns it into a tile id: every
// decision is wave-uniform and the scheduler state lives in scalar registers.
// Only when the current region is exhausted does it steal: it reads all eight
// counters at once (lanes 0-7), picks the first region after the worker's own
// that still has work, claims from it and makes it the current region, so the
// following claims are again a single hidden atomic. A claim that comes back
// out of range proves that region exhausted for good (counters only grow), so
// at most eight steal attempts are made.
// The claim atomic as one assembly statement that skips itself unless `now`
// (wave-uniform) is set: lane 0 alone adds 1 to *ctr (exec is narrowed inside
// the statement) and receives the old value in `ret`. The compiler does not see
// the atomic, so it never waits for it on its own (a claim the compiler could
// see, on any path into the main loop, made it drain every load at the loop
// head): readers of `ret` wait (vmcnt) explicitly. The 16 x 16 main loop sends
// its claims from this statement between two runs of the same loop body, so
// no k-step carries the claim's branch or EXEC write (either one inside the
// step cost 70-90 cycles per step, measured: it holds the wave until the MFMAs
// in flight drain) and no branch splits a step (the register allocator then
// copies accumulators around the split).
__device__ __forceinline__ void claim_issue_asm(uint32_t *ctr, bool now, uint32_t &ret) {
  uint64_t saved;
  asm volatile(
      "s_cmp_eq_u32 %[now], 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "s_mov_b64 %[saved], exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %[ret], %[off], %[one], %[ctr] sc0\n\t"
      "s_mov_b64 exec, %[saved]\n"
      "1:"
      : [ret] "+v"(ret), [saved] "=&s"(saved)
      : [now] "s"(__builtin_amdgcn_readfirstlane(now ? 1u : 0u)), [off] "v"(0u), [one] "v"(1u), [ctr] "s"(ctr)
      : "memory", "scc");
}
__device__ __forceinline__ uint32_t lane0_fetch_add(uint32_t *ctr, uint32_t lane) {
  uint32_t v = 0;
  if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ uint32_t region_size(uint32_t T, uint32_t y) {
  return T > y ? (T - y + kXcdRegions - 1) / kXcdRegions : 0u;
}
// Id of the i-th unit of region y: interleaved regions (policy 1) hold the ids
// 8i + y; contiguous regions (policy 2) hold the y-th of eight consecutive runs
// of ids, of the same sizes (the first T mod 8 runs one longer).
__device__ __forceinline__ uint32_t region_unit(int policy, uint32_t T, uint32_t y, uint32_t i) {
  if (policy == 1) return i * (uint32_t)kXcdRegions + y;
  const uint32_t q = T / (uint32_t)kXcdRegions, r = T % (uint32_t)kXcdRegions;
  return y * q + (y < r ? y : r) + i;
}
__device__ __forceinline__ uint32_t claim_issue(const KernelArgs &a, uint32_t region) {
  uint32_t *ctr = a.claim_policy == 0 ? &a.ctrl->counter : &a.ctrl->xcd_counter[(region) * kXcdStride];
  uint32_t v = 0;
  claim_issue_asm(ctr, true, v);
  return v;
}
__device__ __forceinline__ uint32_t claim_resolve(const KernelArgs &a, uint32_t xcc, uint32_t lane, uint32_t raw,
                                                  uint32_t &region) {
  const uint32_t i0 = __builtin_amdgcn_readfirstlane(raw);
  if (a.claim_policy == 0) return i0 + a.counter_base;
  const uint32_t T = (uint32_t)a.T;
  if (i0 < region_size(T, region)) return region_unit(a.claim_policy, T, region, i0);
  // lane r < 8 watches region (xcc + r) mod 8
  const uint32_t my_y = (xcc + (lane & 7u)) % (uint32_t)kXcdRegions;
  for (int attempt = 0; attempt < kXcdRegions; ++attempt) {
    bool open = false;
    if (lane < (uint32_t)kXcdRegions) {
      const uint32_t seen = __hip_atomic_load(&a.ctrl->xcd_counter[(my_y) * kXcdStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      open = seen < region_size(T, my_y);
    }
    const uint64_t mask = __ballot(open);
    if (mask == 0) return T;
    const uint32_t r = (uint32_t)__builtin_ctzll(mask);
    const uint32_t y = (xcc + r) % (uint32_t)kXcdRegions;
    const uint32_t i = lane0_fetch_add(&a.ctrl->xcd_counter[(y) * kXcdStride], lane);
    if (i < region_size(T, y)) {
      region = y;
      return region_unit(a.claim_policy, T, y, i);
    }
  }
  return T;
}

__device__ __forceinline__ uint32_t claim_next(const KernelArgs &a, uint32_t xcc, uint32_t lane, uint32_t &region) {
  const uint32_t raw = claim_issue(a, region);
  wait_vmem_all();
  return claim_resolve(a, xcc, lane, raw, region);
}

// BT: B is given as N x K row-major (C = A . B^T); its stage then holds BN rows
// x 32 k like A's, and its fragments are read like A's.
template <int BM, int BN, int MODE, bool GROUPED, bool BT>
__global__ __launch_bounds__(TileCfg<BM>::type::THREADS, 1) void ptg_gemm_kernel(const KernelArgs args) {
  using CF = typename TileCfg<BM>::type;
  static_assert(CF::BM_ == BM && CF::BN_ == BN, "config");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[CF::LDS];  // the stage ring
  __shared__ RingRec ring[kRingDepth];
  __shared__ uint32_t gate_ok;
  __shared__ uint32_t split_last;  // this workgroup finished the last K-chunk of a split tile

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = wave_uniform(tid >> 6);
  const uint32_t wm = wave / (uint32_t)CF::WAVES_N_, wn = wave % (uint32_t)CF::WAVES_N_;
  const int32_t T = args.T;

  // ---- clear the next run's scheduler state (spread over the grid)
  if (blockIdx.x == 0 && tid == 0 && args.ctrl_next != nullptr) {
    args.ctrl_next->counter = 0u;
    args.ctrl_next->gate = 0u;
    args.ctrl_next->error = 0u;
    args.ctrl_next->exit_count = 0u;
    for (int x = 0; x < kXcdRegions; ++x) args.ctrl_next->xcd_counter[(x) * kXcdStride] = 0u;
    for (int x = 0; x < kExitGroups; ++x) args.ctrl_next->exit_group[x * kExitStride] = 0u;
  }
  if (args.clear_count > 0) {
    const uint32_t chunk = ((uint32_t)args.clear_count + gridDim.x - 1u) / gridDim.x;
    const uint32_t first = blockIdx.x * chunk;
    for (uint32_t i = tid; i < chunk; i += (uint32_t)CF::THREADS) {
      if (first + i < (uint32_t)args.clear_count) args.clear_next[first + i] = 0u;
    }
  }

  // ---- optional concurrency gate: at most max_concurrent workgroups compute at once
  if (args.max_concurrent > 0) {
    if (tid == 0) {
      // a bounded wait: at most gate_spin_limit polls (the host may preset
      // gate_base slots as taken, so that every wait runs out: failure forcing)
      uint32_t ok = 0;
      for (uint32_t it = 0; it < args.gate_spin_limit; ++it) {
        uint32_t cur = __hip_atomic_load(&args.ctrl->gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cur + args.gate_base < (uint32_t)args.max_concurrent &&
            __hip_atomic_compare_exchange_strong(&args.ctrl->gate, &cur, cur + 1u, __ATOMIC_ACQUIRE,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          ok = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      // a workgroup that gives up computes nothing: its units are lost in the
      // static and non-persistent modes, so the failure is recorded for the host
      if (!ok) flag_error(args, 1u);
      gate_ok = ok;
    }
    __syncthreads();
    if (!gate_ok) {
      if (tid == 0 && args.self_clean) leave_run(args);
      return;
    }
  }

  // scalar reads, kept per wave (only wave 0's values are logged and used to claim)
  const uint32_t hwid = read_hw_id();
  const uint32_t xcc = read_xcc_id() % (uint32_t)kXcdRegions;

  // ---- first work unit (a whole tile, or one K-chunk of a split tile)
  uint32_t ord = 0;       // this worker's unit ordinal
  uint32_t unit = 0;
  bool valid = false;
  // producer state (wave 0, the elected producer, holds the meaningful copy)
  uint32_t next_ord = 1;  // next ordinal to claim
  bool failed = false;    // a claim has come back invalid
  uint32_t region = xcc;  // region the next claim is sent to (XCD-partitioned policy)
  if constexpr (MODE == kDynamic) {
    if (wave == 0) {
      // plain-load pre-check: a slot that starts after every tile was handed
      // out (counters only grow) exits without sending an atomic. Without it,
      // the thousands of late slots of a run with many small tiles sent their
      // atomics to the same counters as the last workers' final claims, whose
      // answers then came back many microseconds late (8192^3 with 128 x 128
      // tiles: 845 -> 955 TFLOP/s). The slots of the first wave (the ones
      // resident at launch) skip it: they start before any claim has gone out,
      // so the counters are open, and the load would only delay their first
      // claim by a round trip. (A first-wave slot that starts late claims
      // anyway, as every slot did before the pre-check.)
      bool open = false;
      if (blockIdx.x < (uint32_t)args.first_wave) {
        open = lane == 0;
      } else if (args.claim_policy != 0) {
        if (lane < (uint32_t)kXcdRegions)
          open = __hip_atomic_load(&args.ctrl->xcd_counter[(lane) * kXcdStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                 region_size((uint32_t)T, lane);
      } else if (lane == 0) {
        open = __hip_atomic_load(&args.ctrl->counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + args.counter_base <
               (uint32_t)T;
      }
      const uint32_t v = __ballot(open) != 0 ? claim_next(args, xcc, lane, region) : (uint32_t)T;
      const uint32_t ok = v < (uint32_t)T ? 1u : 0u;
      if (lane == 0) ring[0] = RingRec{v, ok, 0u, 0u};
      failed = !ok;
    }
    __syncthreads();
    unit = wave_uniform(ring[0].tile);
    valid = wave_uniform(ring[0].valid) != 0;
  } else {
    unit = blockIdx.x;
    valid = unit < (uint32_t)T;
  }

  uint32_t sub = 0;  // the current item's place in its unit (claim groups)
  while (valid) {
    // ---- the work item: unit u covers items [u g, u g + g) (g = claim_group, 1
    // unless claim groups are on); items below split_base are whole tiles (id =
    // tile id), item split_base + q*S + c is K-chunk c of tile split_base + q
    const uint32_t group = (uint32_t)args.claim_group;
    const uint32_t item = unit * group + sub;
    const bool last_sub = sub + 1 >= min(group, (uint32_t)args.items - unit * group);
    uint32_t tile = item;
    uint32_t chunk = 0;
    const bool split = !GROUPED && (int32_t)item >= args.split_base;
    if (split) {
      const uint32_t j = item - (uint32_t)args.split_base;
      tile = (uint32_t)args.split_base + j / (uint32_t)args.split_chunks;
      chunk = j % (uint32_t)args.split_chunks;
    }
    KernelProblem pb;
    int32_t local = (int32_t)tile;
    // what the K-order phase is keyed by: the item (single GEMMs), or the
    // problem (grouped runs: its tiles share its operand panels, so they walk
    // K in step, while different problems take different phases)
    uint32_t rot_key = item;
    if constexpr (GROUPED) {
      const int32_t prob = find_problem(args.groups, args.G, (int32_t)tile);
      rot_key = (uint32_t)prob;
      pb = args.groups[prob];
      // the descriptor is the same for the whole workgroup: keep it in SGPRs
      pb.A = uniform_ptr(pb.A);
      pb.B = uniform_ptr(pb.B);
      pb.C = uniform_ptr(pb.C);
      pb.M = (int32_t)wave_uniform((uint32_t)pb.M);
      pb.N = (int32_t)wave_uniform((uint32_t)pb.N);
      pb.K = (int32_t)wave_uniform((uint32_t)pb.K);
      pb.tiles_m = (int32_t)wave_uniform((uint32_t)pb.tiles_m);
      pb.tiles_n = (int32_t)wave_uniform((uint32_t)pb.tiles_n);
      pb.tile_start = (int32_t)wave_uniform((uint32_t)pb.tile_start);
      pb.unit_start = (int32_t)wave_uniform((uint32_t)pb.unit_start);
      local -= pb.unit_start;
      tile = (uint32_t)(pb.tile_start + local);  // the tile id in call-order numbering
    } else {
      pb = args.single;
    }
    int32_t m_t, n_t;
    decode_tile(local, pb.tiles_m, pb.tiles_n, args.raster_group, m_t, n_t);
    const int32_t m0 = m_t * BM, n0 = n_t * BN;
    const int32_t M = pb.M, N = pb.N, K = pb.K;

    const uint64_t t0 = clock_core();
    const uint64_t r0 = clock_wall();

    // ---- claim ahead (the throttle: at most claims_ahead beyond the current tile)
    uint32_t batch[2] = {0u, 0u};  // raw answers of the claims issued during this tile (lane 0)
    uint32_t batch_ord = 0, batch_n = 0;
    // reserve: the ordinals of the claims this unit sends (wave 0, scalar)
    auto reserve_claims = [&]() {
      if constexpr (MODE == kDynamic) {
        if (wave == 0 && !failed && args.claims_ahead >= 1) {
          batch_ord = next_ord;
          while (next_ord <= ord + (uint32_t)args.claims_ahead && batch_n < 2) {
            ++batch_n;
            ++next_ord;
          }
        }
      }
    };
    // reserve and send at once
    auto do_claims = [&]() {
      if constexpr (MODE == kDynamic) {
        reserve_claims();
        for (uint32_t b = 0; b < batch_n; ++b) {
          const uint32_t v = claim_issue(args, region);
          if (b == 0) batch[0] = v; else batch[1] = v;
        }
      }
    };

    // ---- per-thread load addressing for this tile. Load j of a wave moves a
    // 1 KiB block: A rows (j*NW+wave)*A_RPL .. +A_RPL (A_ROW_CHUNKS lanes per row),
    // B k rows (j*NW+wave)*kBRowsPerLoad .. (B_ROW_CHUNKS lanes per row). Each
    // lane fetches the global chunk whose swizzled slot is its own LDS position.
    // The A swizzle does not change between loads (they step by a multiple of 16
    // rows); the B swizzle flips its bit 1 when a load's k rows step by an odd
    // multiple of 8, so B has two per-lane bases. Each voffset is one of them
    // plus a wave-uniform step.
    constexpr uint32_t kBRowsPerLoad = 64u / CF::B_ROW_CHUNKS;  // k rows one wave-load covers
    constexpr uint32_t kBRowsPerJ = (uint32_t)CF::NW * kBRowsPerLoad;
    const uint32_t a_row0 = wave * (uint32_t)CF::A_RPL + lane / CF::A_ROW_CHUNKS;  // row of load j = a_row0 + RPL NW j
    const uint32_t a_c0 = (lane % CF::A_ROW_CHUNKS) ^ swz_a<CF::MB>(a_row0);
    const uint32_t a_base = a_row0 * (uint32_t)K * 2u;
    const uint32_t b_k0 = wave * kBRowsPerLoad + lane / CF::B_ROW_CHUNKS;  // k row of load j = b_k0 + kBRowsPerJ j
    const uint32_t b_c0 = (lane % CF::B_ROW_CHUNKS) ^ swz_b(b_k0);
    const uint32_t b_c1 = b_c0 ^ 2u;  // the chunk when k row bit 3 is flipped
    const uint32_t b_base0 = n0 + (int32_t)(b_c0 * 8u) < N ? (b_k0 * (uint32_t)N + b_c0 * 8u) * 2u : kBufOob;
    const uint32_t b_base1 = n0 + (int32_t)(b_c1 * 8u) < N ? (b_k0 * (uint32_t)N + b_c1 * 8u) * 2u : kBufOob;
    const int32_t m_left = M - m0;  // rows of A that exist in this tile
    const int32_t n_left = N - n0;  // rows of B^T that exist in this tile (BT)
    const uint16_t *a_tile = pb.A + (size_t)m0 * (size_t)K;
    // the k-step enters through the resource base: + kt BK elements along a row
    // of A (and of B^T), + kt BK rows of B
    const uint16_t *b_tile = BT ? pb.B + (size_t)n0 * (size_t)K : pb.B + n0;
    auto b_kstep = [&](int32_t kt) -> const uint16_t * {
      return BT ? b_tile + kt * CF::BK : b_tile + (size_t)(kt * CF::BK) * (size_t)N;
    };
    const int32_t nk = (K + CF::BK - 1) / CF::BK;
    const int32_t full = K / CF::BK;  // k-steps with no K tail
    // k-steps [kb, ke) of this unit: all of them, or an even share for a K-chunk
    const int32_t kb = split ? (int32_t)((uint32_t)nk * chunk / (uint32_t)args.split_chunks) : 0;
    const int32_t ke = split ? (int32_t)((uint32_t)nk * (chunk + 1u) / (uint32_t)args.split_chunks) : nk;
    // K order of the unit: logical k-step kt (kb <= kt < ke) reads physical k-step
    // kb + ((kt - kb + rot) mod (ke - kb)). When every workgroup walks K from the
    // same end, all concurrent operand reads of the machine share their low
    // address bits (the same 64-byte column of every row of A): measured on a
    // streaming probe of that pattern, 4.5 TB/s against 5.9 TB/s when each CU
    // starts at a different column. A rotation spreads them. It changes only the
    // order of the fp32 sum inside a tile (a function of the unit id alone, so
    // every scheduler still gives bitwise the same C). Off when K has a partial
    // k-step (the K-tail masking assumes that step comes last).
    const int32_t nsteps = ke - kb;
    const int32_t rot = K % CF::BK == 0 ? k_rotation_of(args, rot_key, nsteps) : 0;
    // physical k-step of logical k-step kt (logical steps past ke read zeros
    // through a dead resource, whatever their base)
    auto phys = [&](int32_t kt) -> int32_t { return kt + rot >= ke ? kt + rot - nsteps : kt + rot; };

    // voffset of load j of a k-step with no partial K: chunks outside the matrix
    // (row / column edges) read as zero via kBufOob. The A swizzle of load j's
    // row differs from a_row0's by a compile-time XOR; B has two per-lane bases.
    auto load_chunk_a = [&](int j) -> uint32_t {
      return a_c0 ^ (swz_a<CF::MB>((uint32_t)(CF::A_RPL * CF::NW * j)) ^ swz_a<CF::MB>(0u));
    };
    auto load_voff_edge = [&](int j) -> uint32_t {
      if (j < CF::A_LOADS) {
        const uint32_t row = a_row0 + (uint32_t)(CF::A_RPL * CF::NW) * (uint32_t)j;
        const uint32_t vo = a_base + load_chunk_a(j) * 16u + (uint32_t)(CF::A_RPL * CF::NW * j) * (uint32_t)K * 2u;
        return (int32_t)row >= m_left ? kBufOob : vo;
      }
      const int jb = j - CF::A_LOADS;
      if constexpr (BT) {
        // B^T rows like A rows (same row step per load, same swizzle)
        const uint32_t row = a_row0 + (uint32_t)(CF::A_RPL * CF::NW) * (uint32_t)jb;
        const uint32_t vo = a_row0 * (uint32_t)K * 2u + load_chunk_a(jb) * 16u +
                            (uint32_t)(CF::A_RPL * CF::NW * jb) * (uint32_t)K * 2u;
        return (int32_t)row >= n_left ? kBufOob : vo;
      }
      const uint32_t bb = ((kBRowsPerJ * (uint32_t)jb) & 8u) ? b_base1 : b_base0;
      return bb == kBufOob ? kBufOob : bb + (uint32_t)jb * kBRowsPerJ * (uint32_t)N * 2u;
    };
    // voffset of load j (A loads first, then B) for k-step kt: the same, and in
    // the partial k-step (K tail) chunks past K read as zero too. Every chunk of
    // a k-step past the unit's end reads as zero through its resource (record
    // count 0). The edge offsets do not depend on kt, so the 16 x 16 main loop
    // computes them once per tile and uses them in every trip with no partial
    // K: recomputing the masks every k-step cost about 220 cycles per step in
    // vector instructions interleaved with the MFMAs (measured: 406k -> 350k
    // cycles per 8192^3 tile).
    auto load_voff = [&](int j, int32_t kt) -> uint32_t {
      const uint32_t vo = load_voff_edge(j);
      if (kt < full) return vo;
      const int32_t k0 = kt * CF::BK;
      const int32_t kfirst = j < CF::A_LOADS ? k0 + (int32_t)(load_chunk_a(j) * 8u)
                             : BT ? k0 + (int32_t)(load_chunk_a(j - CF::A_LOADS) * 8u)
                                  : k0 + (int32_t)(b_k0 + kBRowsPerJ * (uint32_t)(j - CF::A_LOADS));
      return kfirst >= K ? kBufOob : vo;
    };
    // LDS byte offset (from smem) of load j's 1 KiB block in stage st
    auto load_dst = [&](int j, int st) -> uint32_t {
      return j < CF::A_LOADS ? (uint32_t)CF::a_off(st) + (uint32_t)(j * CF::NW + (int)wave) * 1024u
                             : (uint32_t)CF::b_off(st) + (uint32_t)((j - CF::A_LOADS) * CF::NW + (int)wave) * 1024u;
    };
    // all loads of k-step kt into stage dst, back to back (prologue)
    auto issue_all = [&](int st, int32_t kt) {
      const i32x4 ra = make_rsrc_words(a_tile + phys(kt) * CF::BK, kt < ke);
      const i32x4 rb = make_rsrc_words(b_kstep(phys(kt)), kt < ke);
      const uint32_t base = lds_addr(smem);
#pragma unroll
      for (int j = 0; j < CF::A_LOADS + CF::B_LOADS; ++j)
        load16_to_lds(j < CF::A_LOADS ? ra : rb, base + load_dst(j, st), load_voff(j, kt));
    };

    // fragment read offsets (bytes inside a stage). An MFMA operand is 8
    // consecutive k per lane: lanes l and l + MB hold the next 8 k of the same
    // row (A) or column (B).
    uint32_t off_a[CF::MI];
    uint32_t swa[CF::MI];
#pragma unroll
    for (int mi = 0; mi < CF::MI; ++mi) {
      const uint32_t row = wm * CF::WM + mi * CF::MB + (lane % CF::MB);
      off_a[mi] = row * (uint32_t)CF::A_ROW;
      swa[mi] = swz_a<CF::MB>(row) ^ (lane / CF::MB);
    }
    uint32_t off_b[CF::NI];
    uint32_t swb[CF::NI];  // BT: the chunk XOR of each block's row, as swa
    if constexpr (BT) {
      // a B^T fragment is read like an A fragment: 8 consecutive k of one row n
#pragma unroll
      for (int ni = 0; ni < CF::NI; ++ni) {
        const uint32_t row = wn * CF::WN + ni * CF::MB + (lane % CF::MB);
        off_b[ni] = row * (uint32_t)CF::A_ROW;
        swb[ni] = swz_a<CF::MB>(row) ^ (lane / CF::MB);
      }
    } else {
      // 32 x 32 blocks: lane group q = lane / 16 covers k half q / 2 and column
      // half q % 2; 16 x 16 blocks: k quarter q of all 16 columns
      const uint32_t q = lane >> 4, i = lane & 15u;
      const uint32_t kk = CF::MB == 32 ? 8u * (q >> 1) + (i >> 2) : 8u * q + (i >> 2);
#pragma unroll
      for (int ni = 0; ni < CF::NI; ++ni) {
        const uint32_t n = CF::MB == 32 ? wn * CF::WN + ni * 32 + 16u * (q & 1u) + 4u * (i & 3u)
                                        : wn * CF::WN + ni * 16 + 4u * (i & 3u);
        off_b[ni] = kk * CF::B_ROW + (((n >> 3) ^ swz_b(kk)) << 4) + ((n & 7u) << 1);
      }
    }

    // A fragment: 8 consecutive k of one row (ds_read_b128). B fragment: two
    // transposing reads of 4 k each (ds_read_b64_tr_b16) for one column. s
    // selects the MFMA's k slice of the stage. Optionally (the 32 x 32 main
    // loop), the loads of k-step kt_load into stage lst are placed in program
    // order between the reads, load j after read j; the reads alternate with
    // MFMAs, so the loads land between MFMAs instead of in one burst. (The
    // 16 x 16 main loop places its reads and loads itself.)
    constexpr int kReads = CF::MI + (BT ? 1 : 2) * CF::NI;
    auto read_frags = [&](int st, int s, bf16x8(&af)[CF::MI], bf16x8(&bfr)[CF::NI], int lst, int32_t kt_load,
                          int count, const uint32_t *voff_fast = nullptr, int j0 = 0) {
      const unsigned char *sa = smem + CF::a_off(st);
      const unsigned char *sb = smem + CF::b_off(st);
      i32x4 ra = {0, 0, 0, 0}, rb = {0, 0, 0, 0};
      const uint32_t lbase = lds_addr(smem);
      if (count > 0) {
        ra = make_rsrc_words(a_tile + phys(kt_load) * CF::BK, kt_load < ke);
        rb = make_rsrc_words(b_kstep(phys(kt_load)), kt_load < ke);
      }
      i16x4 lo[CF::NI];
#pragma unroll
      for (int r = 0; r < kReads; ++r) {
        if (r < CF::MI) {
          af[r] = *(const bf16x8 *)(sa + off_a[r] + ((((uint32_t)((CF::KS / 8) * s)) ^ swa[r]) << 4));
        } else if constexpr (BT) {
          const int ni = r - CF::MI;
          bfr[ni] = *(const bf16x8 *)(sb + off_b[ni] + ((((uint32_t)((CF::KS / 8) * s)) ^ swb[ni]) << 4));
        } else {
          const int ni = (r - CF::MI) >> 1;
          const unsigned char *pb0 = sb + off_b[ni] + (CF::KS * s) * CF::B_ROW;
          if (((r - CF::MI) & 1) == 0) {
            lo[ni] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(pb0));
          } else {
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(pb0 + 4 * CF::B_ROW));
            typedef __attribute__((ext_vector_type(8))) short i16x8;
            const i16x8 v = __builtin_shufflevector(lo[ni], hi, 0, 1, 2, 3, 4, 5, 6, 7);
            bfr[ni] = __builtin_bit_cast(bf16x8, v);
          }
        }
#pragma unroll
        for (int j = 0; j < count; ++j)
          if (j == r)
            load16_to_lds(j0 + j < CF::A_LOADS ? ra : rb, lbase + load_dst(j0 + j, lst),
                          voff_fast ? voff_fast[j0 + j] : load_voff(j0 + j, kt_load));
      }
    };

    typedef float accv __attribute__((ext_vector_type(CF::ACC_N)));
    accv acc[CF::MI][CF::NI];
#pragma unroll
    for (int mi = 0; mi < CF::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < CF::NI; ++ni)
#pragma unroll
        for (int e = 0; e < CF::ACC_N; ++e) acc[mi][ni][e] = 0.0f;

    // the MFMAs of one 16-deep k slice, 32 x 32 blocks (the 16 x 16 main loop
    // issues its own)
    auto mma = [&](const bf16x8(&af)[CF::MI], const bf16x8(&bfr)[CF::NI]) {
      if constexpr (CF::MB == 32) {
#pragma unroll
        for (int mi = 0; mi < CF::MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < CF::NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
    };

    // the prefetch claim is issued claim_lead k-steps before the tile ends (the
    // throttle): late enough not to take work a not-yet-started slot would get,
    // early enough for the atomic's round trip to hide under the MFMAs
    // claims for the next unit go out during the unit's last item only
    const int32_t claim_at = !last_sub ? -1 : ke - kb > args.claim_lead ? ke - args.claim_lead : kb;
    if (ke == kb && last_sub) do_claims();

    constexpr int kLoads = CF::A_LOADS + CF::B_LOADS;
    constexpr int kMfma = CF::MI * CF::NI;
    static_assert(CF::NSTAGE == 4, "stage ring");
    if constexpr (CF::MB == 32) {
      if (ke > kb) {
        // four 32-deep stages: the loads of k-step kt+3 go out during k-step kt
        // into the stage k-step kt-1 just left, so a load has two and a half to
        // three k-steps to land;
        // each k-step is two 16-deep MFMA slices, and the fragments of one slice
        // are read while the other's MFMAs run
        static_assert(kLoads == 4, "stage ring");
        issue_all(0, kb);
        issue_all(1, kb + 1);
        issue_all(2, kb + 2);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        wg_barrier();
        bf16x8 a0[CF::MI], b0[CF::NI], a1[CF::MI], b1[CF::NI];
        read_frags(0, 0, a0, b0, 0, 0, 0);
        // load offsets of a k-step with no partial K, once per tile (as in the
        // 16 x 16 loop); steps whose loads reach the partial k-step `full` use
        // the K-tail test
        uint32_t voff_fast[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) voff_fast[j] = load_voff_edge(j);
        const int32_t slow_from = (K % CF::BK != 0 && full < ke) ? max(kb, full - 3) : ke;
        auto step = [&](int32_t kt, bool fast) {
          const int st = (kt - kb) & 3;
          // two of the four loads of k-step kt+3 go out with each slice's reads
          // (spread over the step: 4096^3 dynamic 175 -> 152 us against all four
          // with the first slice)
          read_frags(st, 1, a1, b1, (st + 3) & 3, kt + 3, kLoads / 2, fast ? voff_fast : nullptr);
          mma(a0, b0);
          interleave<kReads, kMfma>();
          // stage st fully read and stage st+1 landed (its loads went out during
          // step kt-2; the six loads issued since may still be in flight)
          wait_lds_all();
          asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
          wg_barrier();
          read_frags((st + 1) & 3, 0, a0, b0, (st + 3) & 3, kt + 3, kLoads / 2, fast ? voff_fast : nullptr, kLoads / 2);
          mma(a1, b1);
          interleave<kReads, kMfma>();
        };
        int32_t kt = kb;
        auto steps = [&](int32_t end) {
          for (const int32_t fe = min(end, slow_from); kt < fe; ++kt) step(kt, true);
          for (; kt < end; ++kt) step(kt, false);
        };
        // the claims go out between two runs of the loop (no branch for them in a step)
        if constexpr (MODE == kDynamic) {
          steps(claim_at >= kb ? claim_at : ke);
          if (claim_at >= kb) do_claims();
        }
        steps(ke);
      }
    } else {
      if (ke > kb) {
        // four 32-deep stages, one 32-deep MFMA per block and k-step: the
        // fragments of k-step kt+1 are read from its stage while step kt's MFMAs
        // run on the fragments read during step kt-1. The loads of step kt+4 go
        // out during step kt into the stage step kt's fragments came from (every
        // wave finished reading it before the barrier that ended step kt-1), and
        // must have landed by the barrier that ends step kt+2: between two and
        // three k-steps in flight.
        static_assert(kLoads == 8, "stage ring");
        issue_all(0, kb);
        issue_all(1, kb + 1);
        issue_all(2, kb + 2);
        issue_all(3, kb + 3);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // stages 0 and 1 landed
        wg_barrier();
        bf16x8 a0[CF::MI], b0[CF::NI], a1[CF::MI], b1[CF::NI];
        read_frags(0, 0, a0, b0, 0, 0, 0);
        wait_lds_all();
        wg_barrier();  // stage 0 read by every wave before step kb's loads refill it
        // claims are reserved now and sent between the two loop runs below
        if (claim_at >= 0) reserve_claims();
        uint32_t *claim_ctr = args.claim_policy == 0 ? &args.ctrl->counter : &args.ctrl->xcd_counter[(region) * kXcdStride];
        // The MFMA as a statement of its own, accumulating in place: each of the
        // 64 accumulators keeps one AGPR quad for the whole loop (all 256 AGPRs
        // hold accumulators, and with the builtin the register allocator
        // rotated some through copies every trip). The statements are volatile
        // and clobber memory, so program order is issue order: MFMA i, then
        // fragment read i of the next k-step (24 reads), and the eight loads
        // of k-step kt + 4 after MFMAs 3, 10, ..., 52 (one every seven: spread
        // over the step, they hold the MFMA stream least; measured against one
        // after every third read, 302k against 317k cycles per 8192^3 tile and
        // 3-4% off the HBM-bound shapes; all eight together after the first
        // MFMA cost 392k). Hazards: within the loop the MFMA operands are
        // written only by LDS reads (waited for), and accumulators are written
        // only by MFMAs; the fences before and after the loop give the wait
        // states the compiler cannot see.
        auto mfma16 = [&](int mi, int ni, const bf16x8 &a, const bf16x8 &b) {
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[mi][ni]) : "v"(b), "v"(a) : "memory");
        };
        // per-lane load offsets of a k-step with no partial K (see load_voff_edge)
        uint32_t voff_fast[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) voff_fast[j] = load_voff_edge(j);
        // FAST: the k-step's loads read whole 32-deep slices (or lie past the
        // unit and read zeros through the resource), so the offsets above serve;
        // otherwise they are computed with the K-tail test.
        // st: the stage step kt's fragments came from, (kt - kb) mod 4; a compile-time
        // constant in the four-step trips, so every LDS address of the step is a
        // per-lane base plus an immediate offset
        auto step = [&](auto fast, int32_t kt, int st, const bf16x8(&ac)[CF::MI], const bf16x8(&bc)[CF::NI],
                        bf16x8(&an)[CF::MI], bf16x8(&bn)[CF::NI]) {
          const int rst = (st + 1) & 3;
          const unsigned char *sa = smem + CF::a_off(rst);
          const unsigned char *sb = smem + CF::b_off(rst);
          const int32_t kt_load = kt + 4;
          const i32x4 ra = make_rsrc_words(a_tile + phys(kt_load) * CF::BK, kt_load < ke);
          const i32x4 rb = make_rsrc_words(b_kstep(phys(kt_load)), kt_load < ke);
          const uint32_t lbase = lds_addr(smem);
          i16x4 lo[CF::NI];
#pragma unroll
          for (int i = 0; i < kMfma; ++i) {
            mfma16(i / CF::NI, i % CF::NI, ac[i / CF::NI], bc[i % CF::NI]);
            if (i < kReads) {
              const int r = i;
              if (r < CF::MI) {
                an[r] = *(const bf16x8 *)(sa + off_a[r] + (swa[r] << 4));
              } else if constexpr (BT) {
                bn[r - CF::MI] = *(const bf16x8 *)(sb + off_b[r - CF::MI] + (swb[r - CF::MI] << 4));
              } else {
                const int ni = (r - CF::MI) >> 1;
                const unsigned char *pb0 = sb + off_b[ni];
                if (((r - CF::MI) & 1) == 0) {
                  lo[ni] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(pb0));
                } else {
                  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(pb0 + 4 * CF::B_ROW));
                  typedef __attribute__((ext_vector_type(8))) short i16x8;
                  const i16x8 v = __builtin_shufflevector(lo[ni], hi, 0, 1, 2, 3, 4, 5, 6, 7);
                  bn[ni] = __builtin_bit_cast(bf16x8, v);
                }
              }
            }
            // (a spacing of eight, which lines the loads up with the rows of the
            // accumulator grid, made the compiler give up unrolling the step)
            static_assert(3 + 7 * (kLoads - 1) < kMfma, "load placement");
#pragma unroll
            for (int j = 0; j < kLoads; ++j)
              if (3 + 7 * j == i)
                load16_to_lds(j < CF::A_LOADS ? ra : rb, lbase + load_dst(j, st),
                              decltype(fast)::value ? voff_fast[j] : load_voff(j, kt_load));
          }
          wait_lds_all();
          asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
          wg_barrier();
        };
        // the zeroed accumulators in their registers, then 16 wait states, before
        // the first MFMA reads them
#pragma unroll
        for (int mi = 0; mi < CF::MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < CF::NI; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
        // two steps per trip, so the fragment buffers swap roles by name. An odd
        // count ends with one step past the unit: its stage was zero-filled, and
        // adding zero products leaves every accumulator bit for bit as it was.
        // The dynamic scheduler runs the loop in two parts and sends its claims
        // between them, at the trip boundary at or before claim_at.
        // Trips whose loads reach the partial k-step `full` (K not a multiple of
        // 32, and the unit ends after it) use the K-tail test: from the first trip
        // t (t - kb even) with t + 5 >= full on; the trips before it use the fast
        // offsets.
        const int32_t slow_from =
            (K % CF::BK != 0 && full < ke) ? kb + ((max(full - 5 - kb, 0) + 1) / 2) * 2 : ke + 2;
        // Fast trips of four steps while whole ones fit (constant stages), then
        // two-step trips with the stage computed at run time. A run starts with
        // kt - kb a multiple of 4.
        auto trips = [&](int32_t &kt, int32_t end) {
          const int32_t fast_end = min(end, slow_from);
          for (; kt + 4 <= fast_end; kt += 4) {
            step(std::true_type{}, kt, 0, a0, b0, a1, b1);
            step(std::true_type{}, kt + 1, 1, a1, b1, a0, b0);
            step(std::true_type{}, kt + 2, 2, a0, b0, a1, b1);
            step(std::true_type{}, kt + 3, 3, a1, b1, a0, b0);
          }
          for (; kt < fast_end; kt += 2) {
            const int st = (kt - kb) & 3;
            step(std::true_type{}, kt, st, a0, b0, a1, b1);
            step(std::true_type{}, kt + 1, (st + 1) & 3, a1, b1, a0, b0);
          }
          for (; kt < end; kt += 2) {
            const int st = (kt - kb) & 3;
            step(std::false_type{}, kt, st, a0, b0, a1, b1);
            step(std::false_type{}, kt + 1, (st + 1) & 3, a1, b1, a0, b0);
          }
        };
        int32_t kt = kb;
        if constexpr (MODE == kDynamic) {
          // the claims go out at the four-step boundary at or before claim_at
          const int32_t split_at = claim_at >= kb ? kb + ((claim_at - kb) & ~3) : ke;
          trips(kt, split_at);
          claim_issue_asm(claim_ctr, batch_n >= 1u, batch[0]);
          claim_issue_asm(claim_ctr, batch_n >= 2u, batch[1]);
        }
        trips(kt, ke);
        // 24 wait states after the last MFMA before anything reads an accumulator
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int mi = 0; mi < CF::MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < CF::NI; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
      }
    }

    // ---- publish the claims issued during this unit (producer, wave 0): each
    // answer goes to its ring record. Prefetch claims are resolved here, before
    // the epilogue: reading an atomic's answer waits for every older memory
    // operation of the wave, and the C stores would otherwise be among them.
    auto publish_claims = [&]() {
      // the answers of claims sent from assembly. A full drain: a returning
      // atomic is not ordered with the loads issued after it, so only vmcnt 0
      // proves its answer (and the register it writes) has arrived
      wait_vmem_all();
      for (uint32_t b = 0; b < batch_n; ++b) {
        const uint32_t v = claim_resolve(args, xcc, lane, b == 0 ? batch[0] : batch[1], region);
        const uint32_t ok = v < (uint32_t)T ? 1u : 0u;
        if (!ok) failed = true;
        if (lane == 0) ring[(batch_ord + b) % (uint32_t)args.ring_depth] = RingRec{v, ok, batch_ord + b, 0u};
      }
    };
    // With claims sent during the unit, the next unit's record is read right
    // after they are published, so the end of the unit needs no barrier.
    RingRec next_rec = RingRec{0u, 0u, 0u, 0u};
    bool next_read = false;
    if constexpr (MODE == kDynamic) {
      if (args.claims_ahead >= 1) {
        if (wave == 0) publish_claims();
        if (last_sub) {
          __syncthreads();
          next_rec = ring[(ord + 1) % (uint32_t)args.ring_depth];
          next_read = true;
        }
      }
    }

    // ---- epilogue: fp32 accumulators -> C. Lane l holds, in each group of four
    // accumulators, 4 consecutive n of row m = l % MB of its block: n = 8 qd +
    // 4 (l / 32) for 32 x 32 blocks, 4 (l / 16) for 16 x 16 blocks; group g =
    // (mi NI + ni) QUADS + qd of a thread is its g-th group. C is written once
    // and never read by the kernel, so the stores are non-temporal: they do not
    // displace the A and B slices the XCD's other workgroups are still reading
    // from L2 (measured 1-3% faster across the modes).
    const bool interior = m0 + BM <= M && n0 + BN <= N;

    // Whole rows per store. Written straight from the accumulators, one store
    // covers 16 rows x 64 B (16 x 16 blocks) or 32 rows x 32 B (32 x 32
    // blocks), and a CU then writes a 256 KiB tile in about 7 us whether or not
    // other CUs store too (measured with a store-only kernel), while stores of
    // whole rows take about 2 us alone and reach about 8 TB/s when every CU
    // stores at once. So each wave passes its WM x WN results through its
    // quarter of the stage ring, RP rows (a pass) at a time, and reads them back
    // a row at a time: each store then writes RPR rows of WN contiguous floats.
    // 16-byte chunk c of row r sits in slot c ^ (r mod 16), which keeps the
    // block-shaped writes and the row-shaped reads free of bank conflicts.
    // epi_begin / epi_end bracket the use of the ring (every wave calls them);
    // stage writes a group of four results of pass p, flush stores pass p.
    constexpr int WAVE_LDS = CF::LDS / CF::NW;
    constexpr int ROW_B = CF::WN * 4;
    constexpr int RP = WAVE_LDS / ROW_B < CF::WM ? WAVE_LDS / ROW_B : CF::WM;
    constexpr int CHUNKS = ROW_B / 16;
    constexpr int RPR = 1024 / ROW_B;
    constexpr int MI_PASS = RP / CF::MB;
    constexpr int PASSES = CF::WM / RP;
    static_assert(CF::WM % RP == 0 && RP % CF::MB == 0 && CHUNKS * RPR == 64 && CHUNKS <= 32, "epilogue");
    unsigned char *wl = smem + wave * WAVE_LDS;
    auto epi_begin = [&]() {
      // every wave's loads into the stages have landed and its fragment reads
      // are done before any wave overwrites the stages
      wait_vmem_all();
      wg_barrier();
    };
    auto stage = [&](int p, int mi, int ni, int qd, const f32x4 &v) {
      const uint32_t row = (uint32_t)((mi - p * MI_PASS) * CF::MB) + lane % CF::MB;
      const uint32_t c = (uint32_t)(ni * (CF::MB / 4) + 2 * qd) + lane / CF::MB;
      *(f32x4 *)(wl + row * ROW_B + ((c ^ (row & 15u)) << 4)) = v;
    };
    auto flush = [&](int p) {
      // the wave's own LDS writes complete before its reads of other lanes' data
      wait_lds_all();
      __builtin_amdgcn_wave_barrier();
#pragma unroll 4
      for (int i = 0; i < RP / RPR; ++i) {
        const uint32_t row = (uint32_t)(i * RPR) + lane / CHUNKS;
        const uint32_t c = lane % CHUNKS;
        const f32x4 v = *(const f32x4 *)(wl + row * ROW_B + ((c ^ (row & 15u)) << 4));
        const int32_t m = m0 + (int32_t)(wm * CF::WM + p * RP + row);
        const int32_t n = n0 + (int32_t)(wn * CF::WN + 4 * c);
        if (interior || (m < M && n < N)) __builtin_nontemporal_store(v, (f32x4 *)(pb.C + (size_t)m * (size_t)N + n));
      }
      // the reads are done before the next pass (or the next unit's loads) writes the region
      wait_lds_all();
      __builtin_amdgcn_wave_barrier();
    };
    auto epi_end = [&]() { wg_barrier(); };

    if (!split) {
      epi_begin();
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
#pragma unroll
        for (int mi = p * MI_PASS; mi < (p + 1) * MI_PASS; ++mi)
#pragma unroll
          for (int ni = 0; ni < CF::NI; ++ni)
#pragma unroll
            for (int qd = 0; qd < CF::QUADS; ++qd)
              stage(p, mi, ni, qd, f32x4{acc[mi][ni][4 * qd + 0], acc[mi][ni][4 * qd + 1], acc[mi][ni][4 * qd + 2],
                                         acc[mi][ni][4 * qd + 3]});
        flush(p);
      }
      epi_end();
    } else {
      // K-chunk of a split tile: publish the partial sum; the workgroup that
      // completes the tile's last chunk adds all partials in chunk order and
      // writes C. The order is fixed, so the result does not depend on who
      // finished last. Partial slots are thread-major per 16-byte group: fully
      // coalesced. The sum reads the other chunks' slots in batches of up to
      // 16 groups per thread, all of a chunk's loads of a batch in flight at once.
      // The partials are written and read with agent-scope cache policy
      // (store16_agent / load16_agent): the stores go through to memory and a
      // vmcnt(0) wait completes them before the arrival count goes out, so the
      // count itself can be relaxed. Release and acquire fences in their place
      // write back and invalidate the whole L2 of the XCD; with every tile of a
      // run split (fewer tiles than workers) they cost 2048 x 2048 x 8192 about
      // a third of its time.
      const uint32_t S = (uint32_t)args.split_chunks;
      const uint32_t q = tile - (uint32_t)args.split_base;
      const __amdgpu_buffer_rsrc_t wsr = make_rsrc(args.ws);
      const uint32_t slot_off = (item - (uint32_t)args.split_base) * (uint32_t)(BM * BN * 4);
#pragma unroll
      for (int mi = 0; mi < CF::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < CF::NI; ++ni)
#pragma unroll
          for (int qd = 0; qd < CF::QUADS; ++qd) {
            const int g = (mi * CF::NI + ni) * CF::QUADS + qd;
            store16_agent(wsr, slot_off + (uint32_t)(g * CF::THREADS + (int)tid) * 16u,
                          f32x4{acc[mi][ni][4 * qd + 0], acc[mi][ni][4 * qd + 1], acc[mi][ni][4 * qd + 2],
                                acc[mi][ni][4 * qd + 3]});
          }
      wait_vmem_all();  // this thread's partial has reached memory
      __syncthreads();
      if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&args.arrivals[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        split_last = prev + 1u == S ? 1u : 0u;
        // every chunk has arrived: the count is done with for this run
        if (prev + 1u == S) __hip_atomic_store(&args.arrivals[q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (wave_uniform(split_last) != 0) {
        // the sum in chunk order, staged straight into the ring a pass at a
        // time and stored in whole rows like a whole tile (the partial loads
        // go out after the count's answer, which every thread has waited for)
        const uint32_t base = q * S * (uint32_t)(BM * BN * 4) + tid * 16u;
        constexpr int kPassGroups = MI_PASS * CF::NI * CF::QUADS;  // groups g of pass p: p kPassGroups + [0, kPassGroups)
        constexpr int kBatch = kPassGroups < 16 ? kPassGroups : 16;
        static_assert(kPassGroups % kBatch == 0, "batches");
        epi_begin();
        for (int p = 0; p < PASSES; ++p) {
          for (int g0 = p * kPassGroups; g0 < (p + 1) * kPassGroups; g0 += kBatch) {
            f32x4 v[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) v[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            for (uint32_t c = 0; c < S; ++c) {
              const uint32_t src = base + c * (uint32_t)(BM * BN * 4) + (uint32_t)(g0 * CF::THREADS) * 16u;
              f32x4 part[kBatch];
#pragma unroll
              for (int i = 0; i < kBatch; ++i) part[i] = load16_agent(wsr, src + (uint32_t)(i * CF::THREADS) * 16u);
#pragma unroll
              for (int i = 0; i < kBatch; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) v[i][e] += part[i][e];
            }
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
              const int g = g0 + i;
              stage(p, g / (CF::NI * CF::QUADS), (g / CF::QUADS) % CF::NI, g % CF::QUADS, v[i]);
            }
          }
          flush(p);
        }
        epi_end();
      }
    }

    // ---- claims after the work (claims_ahead = 0): issue and publish
    if (wave == 0) {
      if constexpr (MODE == kDynamic) {
        if (args.claims_ahead == 0 && !failed && last_sub) {
          batch_ord = next_ord;
          batch[0] = claim_issue(args, region);
          batch_n = 1;
          ++next_ord;
          publish_claims();
        }
      }
    }
    // ---- log the tile
    if (tid == 0) {
      const uint64_t t1 = clock_core();
      const uint64_t r1 = clock_wall();
      if ((int32_t)item < args.log_cap) {
        TileRecDev rec;
        rec.tile = tile;
        rec.unit = unit;
        rec.pad = 0;
        rec.kb = (uint32_t)kb;
        rec.ke = (uint32_t)ke;
        rec.worker = blockIdx.x;
        rec.hw_id = hwid;
        rec.xcc_id = xcc;
        rec.t0 = t0;
        rec.t1 = t1;
        rec.r0 = r0;
        rec.r1 = r1;
        args.log[item] = rec;
        __hip_atomic_fetch_add(&args.visits[item], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---- advance: the next item of this unit, else the next unit
    if (!last_sub) {
      ++sub;
      continue;
    }
    sub = 0;
    if constexpr (MODE == kDynamic) {
      if (!next_read) {
        __syncthreads();
        next_rec = ring[(ord + 1) % (uint32_t)args.ring_depth];
      }
      const RingRec rec = next_rec;
      const uint32_t seq = wave_uniform(rec.seq);
      valid = wave_uniform(rec.valid) != 0;
      unit = wave_uniform(rec.tile);
      if (seq != ord + 1) {
        // the ring protocol was violated: stop this worker and flag it
        if (tid == 0) flag_error(args, 2u);
        valid = false;
      }
    } else if constexpr (MODE == kStatic) {
      unit += (uint32_t)args.P;
      valid = unit < (uint32_t)T;
    } else {
      valid = false;
    }
    ++ord;
  }

  if (tid == 0) {
    if (args.max_concurrent > 0)
      __hip_atomic_fetch_sub(&args.ctrl->gate, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (args.self_clean) leave_run(args);
  }
}

template <int BM, int BN, int MODE, bool GROUPED, bool BT>
static hipError_t launch_one(const KernelArgs &args, int grid, int dyn_lds, hipStream_t stream) {
  hipLaunchKernelGGL((ptg_gemm_kernel<BM, BN, MODE, GROUPED, BT>), dim3(grid), dim3(TileCfg<BM>::type::THREADS),
                     dyn_lds, stream, args);
  return hipGetLastError();
}

template <int BM, int BN, bool BT>
static hipError_t launch_tile(int mode, bool grouped, const KernelArgs &args, int grid, int dyn_lds,
                              hipStream_t stream) {
  switch (mode) {
    case kNonPersistent:
      return grouped ? launch_one<BM, BN, kNonPersistent, true, BT>(args, grid, dyn_lds, stream)
                     : launch_one<BM, BN, kNonPersistent, false, BT>(args, grid, dyn_lds, stream);
    case kStatic:
      return grouped ? launch_one<BM, BN, kStatic, true, BT>(args, grid, dyn_lds, stream)
                     : launch_one<BM, BN, kStatic, false, BT>(args, grid, dyn_lds, stream);
    case kDynamic:
      return grouped ? launch_one<BM, BN, kDynamic, true, BT>(args, grid, dyn_lds, stream)
                     : launch_one<BM, BN, kDynamic, false, BT>(args, grid, dyn_lds, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int tile_edge, int mode, bool grouped, bool b_transposed, const KernelArgs &args, int grid,
                       int dyn_lds, hipStream_t stream) {
  if (tile_edge == 256)
    return b_transposed ? launch_tile<256, 256, true>(mode, grouped, args, grid, dyn_lds, stream)
                        : launch_tile<256, 256, false>(mode, grouped, args, grid, dyn_lds, stream);
  if (tile_edge == 128)
    return b_transposed ? launch_tile<128, 128, true>(mode, grouped, args, grid, dyn_lds, stream)
                        : launch_tile<128, 128, false>(mode, grouped, args, grid, dyn_lds, stream);
  return hipErrorInvalidValue;
}

hipError_t gemm_occupancy(int tile_edge, int dyn_lds, int *blocks_per_cu) {
  if (tile_edge == 256)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, reinterpret_cast<const void *>(&ptg_gemm_kernel<256, 256, kDynamic, false, false>),
        TileCfg<256>::type::THREADS, dyn_lds);
  if (tile_edge == 128)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, reinterpret_cast<const void *>(&ptg_gemm_kernel<128, 128, kDynamic, false, false>),
        TileCfg<128>::type::THREADS, dyn_lds);
  return hipErrorInvalidValue;
}

int gemm_static_lds_bytes(int tile_edge) {
  if (tile_edge == 256) return TileCfg<256>::type::LDS + (int)sizeof(RingRec) * kRingDepth + 4;
  if (tile_edge == 128) return TileCfg<128>::type::LDS + (int)sizeof(RingRec) * kRingDepth + 4;
  return 0;
}

}  // namespace ptg

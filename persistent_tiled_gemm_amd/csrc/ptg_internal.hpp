// Types shared by the host library and the kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptg {

// One GEMM problem as the kernel sees it. Grouped launches pass an array of
// these in device memory; a single GEMM passes one by value.
struct KernelProblem {
  const uint16_t *A;   // M x K bf16 bits, row-major
  const uint16_t *B;   // K x N bf16 bits, row-major
  float *C;            // M x N fp32, row-major
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t tile_start;  // first global tile id of this problem (problems numbered in call order)
  int32_t unit_start;  // first work unit of this problem (units numbered in claim order)
};

// Tile regions of the XCD-partitioned claim policy: region x holds the tiles
// with id mod kXcdRegions == x (MI355X has 8 XCDs; workgroup w runs on XCD w mod 8).
static constexpr int kXcdRegions = 8;

// Scheduler state in device memory. A plan keeps three sets (control block +
// split arrival and visit counters): uncaptured run i uses set i % 2 and clears
// set (i + 1) % 2 for the next run, so a run is exactly one kernel launch with
// no host-side reset. A launch captured into a graph uses the third set and
// leaves its counters at zero itself (self_clean: the last workgroup to finish
// resets them; the last chunk of a split tile always resets its arrival
// count), so the launch replayed again and again on that set starts clean.
// Workgroups count themselves out of a run in kExitGroups groups (workgroup w
// in group w mod kExitGroups), each group's count on a cache line of its own:
// thousands of late launch slots leaving at once serialise on one counter.
static constexpr int kExitGroups = 16;
static constexpr int kExitStride = 32;  // u32 words from one group's count to the next (128 bytes)

// The per-XCD claim counters sit kXcdStride words (256 bytes) apart: with all
// eight in one cache line, the claims of every XCD queued on that line
// (measured: 4096^3 with 128 x 128 tiles, 512 workers, dynamic 156.5 -> 152.3
// us; no change with 256 x 256 tiles).
static constexpr int kXcdStride = 64;

struct alignas(128) SchedCtrl {
  uint32_t counter;    // dynamic claim counter (single-counter policy)
  uint32_t gate;       // workgroups currently holding a concurrency slot
  uint32_t error;      // bit 0: a gate wait ran out; bit 1: ring record for the wrong ordinal
  uint32_t exit_count; // exit groups whose workgroups have all finished (the last group resets the counters)
  uint32_t pad[28];
  uint32_t xcd_counter[kXcdRegions * kXcdStride];  // per-XCD claim counters at [x * kXcdStride] (XCD-partitioned policy)
  uint32_t exit_group[kExitGroups * kExitStride];  // group g's finished workgroups at [g * kExitStride]
};
static_assert(sizeof(SchedCtrl) == 128 + 4 * kXcdStride * kXcdRegions + 128 * kExitGroups, "control block layout");

// Most tiles one run may split along K (the partial last wave); each has an
// arrival counter in the scheduler-state set.
static constexpr int kMaxSplitTiles = 1024;

// Log record as written by the kernel, one per work item (a whole tile or one
// K-chunk of a split tile), indexed by item id. unit: the claimed work unit that
// covered the item (items are units unless claim groups are on); kb / ke: the
// item's k-steps [kb, ke) of BK each.
struct TileRecDev {
  uint32_t tile, worker, hw_id, xcc_id;
  uint64_t t0, t1, r0, r1;
  uint32_t kb, ke, unit, pad;
};
static_assert(sizeof(TileRecDev) == 64, "tile record layout");

struct KernelArgs {
  KernelProblem single;         // the problem when G == 1 and !grouped
  const KernelProblem *groups;  // device array (grouped launches)
  int32_t G;
  int32_t T;                    // work units handed out (claims, static steps, non-persistent blocks)
  int32_t items;                // work items: tiles, plus the K-chunks of split tiles
  int32_t claim_group;          // items per unit (1 unless claim groups are on; then nothing is split)
  int32_t split_base;           // items >= split_base are K-chunks of the tiles split_base, ...; == items: no split
  int32_t split_chunks;         // K-chunks per split tile (S)
  float *ws;                    // split partial sums: one BM x BN fp32 slot per K-chunk item
  uint32_t *arrivals;           // this run's per-split-tile arrival counters (kMaxSplitTiles)
  int32_t P;                    // static stride (grid size of a static run)
  int32_t claims_ahead;         // 0, 1 or 2 (< ring_depth)
  int32_t ring_depth;           // 2 or 3
  int32_t claim_lead;           // prefetch claims are issued this many k-steps before a tile ends
  int32_t claim_policy;         // 0: one global counter; 1/2: per-XCD counters (interleaved / contiguous regions) with stealing
  int32_t raster_group;         // <= 1: row-major
  int32_t k_rotation;           // K order per unit: 0 = kb..ke-1; rotated by a phase per XCD region (1), two per region (2), per unit (3)
  uint32_t counter_base;        // added to every claim (failure forcing)
  int32_t max_concurrent;       // 0: no gate
  uint32_t gate_spin_limit;     // polls of the gate before a workgroup gives up (> 0)
  uint32_t gate_base;           // gate slots taken before the run starts (failure forcing; normally 0)
  uint32_t *status;             // the plan's sticky device status: error bits of every run since the host last read it
  int32_t log_cap;              // items logged (0: none)
  SchedCtrl *ctrl;              // this run's set
  TileRecDev *log;
  uint32_t *visits;
  SchedCtrl *ctrl_next;         // the next run's set, cleared by this run
  uint32_t *clear_next;         // the next set's arrival + visit counters (contiguous)
  int32_t clear_count;          // counters to clear there
  int32_t first_wave;           // dynamic: slots below this index claim without the pre-check (those resident at launch)
  int32_t self_clean;           // 1: the run leaves its set at zero when it ends (captured launches, which
                                // replay on one set); 0: the next run clears the set instead
};

enum SchedMode { kNonPersistent = 0, kStatic = 1, kDynamic = 2 };

// Launch one GEMM kernel instance. tile_edge is 128 or 256; b_transposed: B is
// given as N x K row-major (C = A . B^T) instead of K x N.
hipError_t launch_gemm(int tile_edge, int mode, bool grouped, bool b_transposed, const KernelArgs &args, int grid,
                       int dyn_lds_bytes, hipStream_t stream);
// Resident workgroups per CU for an instance with dyn_lds_bytes of extra LDS.
hipError_t gemm_occupancy(int tile_edge, int dyn_lds_bytes, int *blocks_per_cu);
// Static LDS of an instance, bytes.
int gemm_static_lds_bytes(int tile_edge);

hipError_t launch_spoiler(int n_wgs, uint64_t spin_ticks, uint32_t *resident, uint64_t *log, hipStream_t stream);

// MFMA-only probe: `grid` workgroups of four waves, `iters` rounds per wave of
// eight 32x32x16 (mfma_block 32) or sixteen 16x16x32 (mfma_block 16) bf16
// MFMAs; ticks receives {s_memtime, s_memrealtime} deltas per workgroup.
hipError_t launch_mfma_probe(int grid, int32_t iters, bool vary, int mfma_block, float *sink, uint64_t *ticks,
                             hipStream_t s);

}  // namespace ptg

// Host side of the C ABI declared in include/ptg_gemm.h: plan creation and
// validation, launch sizing per scheduler, per-run scratch reset, tile-log
// and device-status readback, the spoiler, CU-masked streams and the
// failure-forcing helpers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "ptg_gemm.h"
#include "ptg_internal.hpp"

namespace ptg {
// Memory-only probe (hbm_probe.hip): kind 0 reads `bytes` of src (zeros) into a
// sum, kind 1 copies `bytes` from src to dst; `grid` workgroups of 256 threads,
// 16 bytes per lane.
hipError_t launch_hbm_probe(int kind, int grid, const void *src, void *dst, size_t bytes, float *sink,
                            hipStream_t s);
}  // namespace ptg

using ptg::KernelArgs;
using ptg::KernelProblem;
using ptg::SchedCtrl;
using ptg::TileRecDev;

struct gemm_plan {
  gemm_tile_desc desc;
  int cu_count = 0;
  int occupancy = 0;
  int static_workers = 0;
  int64_t wallclock_khz = 0;
  int lds_bytes = 0;
  int dyn_lds = 0;
  // device scratch: three sets of [SchedCtrl][arrivals u32 x kMaxSplitTiles][visits u32 x
  // log_capacity] (two for uncaptured runs, one for captured launches) followed by
  // the sticky status word, plus the log and (tail
  // splitting on) the partial-sum workspace
  unsigned char *d_ctrl_block = nullptr;
  uint32_t *d_status = nullptr;  // error bits of every run since the host last read them
  float *d_ws = nullptr;
  int64_t ws_tiles = 0;  // BM x BN fp32 partial slots in d_ws
  size_t ctrl_set_bytes = 0;
  uint64_t runs = 0;  // uncaptured launches so far; run i uses set i % 2
  unsigned char *last_set = nullptr;  // the state set of the last launch (its visit counters)
  TileRecDev *d_log = nullptr;
  KernelProblem *d_groups = nullptr;
  KernelProblem *h_groups = nullptr;  // pinned staging for the grouped table
  hipEvent_t groups_uploaded = nullptr;
  bool groups_event_pending = false;
  std::vector<KernelProblem> last_groups;  // what d_groups holds
  uint32_t preset = 0;
  bool preset_pending = false;
  uint32_t gate_preset = 0;
  bool gate_preset_pending = false;
  hipEvent_t stream_switch = nullptr;  // orders a run on a new stream after the plan's last stream
  // last run
  hipStream_t last_stream = nullptr;
  bool has_run = false;
  int64_t last_tiles = 0;
  int64_t last_units = 0;
  int64_t last_items = 0;
  int64_t last_split_base = 0;
  int32_t last_split_chunks = 0;
  int32_t last_claim_group = 1;
  int64_t last_grid = 0;
  int32_t last_mode = -1;
  int32_t last_k_rotation = GEMM_KROT_OFF;
  std::vector<int32_t> last_tile_start;  // per problem (grouped), for log decoding
  std::vector<int32_t> last_k;           // K per problem, for log decoding
  std::vector<std::pair<int32_t, int32_t>> last_unit_map;  // grouped, claim order: (unit_start, tile_start)
  std::string last_error;
};

namespace {

gemm_status hip_fail(gemm_plan *p, hipError_t e, const char *what) {
  if (p) {
    p->last_error = std::string(what) + ": " + hipGetErrorString(e);
  }
  return GEMM_E_HIP;
}

bool valid_tile(const gemm_tile_desc &d) {
  return (d.bm == 256 && d.bn == 256 && d.bk == 32) || (d.bm == 128 && d.bn == 128 && d.bk == 32);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

gemm_status check_problem(const void *A, const void *B, const float *C, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return GEMM_E_SHAPE;
  if (M > GEMM_MAX_M || N > GEMM_MAX_N || K > GEMM_MAX_K) return GEMM_E_SHAPE;
  if ((N % 8) != 0 || (K % 8) != 0) return GEMM_E_SHAPE;
  if (M == 0 || N == 0) return GEMM_OK;
  if (C == nullptr) return GEMM_E_INVALID_ARG;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_E_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) | reinterpret_cast<uintptr_t>(C)) & 15u)
    return GEMM_E_INVALID_ARG;
  return GEMM_OK;
}

gemm_status check_current_device(gemm_plan *p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(p, e, "hipGetDevice");
  if (dev != p->desc.device) return GEMM_E_DEVICE;
  return GEMM_OK;
}

// A plan's scratch (scheduler state, grouped table, split workspace) is used by
// one run at a time. Runs on one stream are ordered by the stream; a run on a
// different stream than the last one first waits (on the device) for
// everything enqueued on the last stream so far. No host synchronisation.
gemm_status order_after_last_stream(gemm_plan *p, hipStream_t s) {
  if (!p->has_run || s == p->last_stream) return GEMM_OK;
  hipError_t e = hipEventRecord(p->stream_switch, p->last_stream);
  if (e != hipSuccess) return hip_fail(p, e, "hipEventRecord(stream switch)");
  e = hipStreamWaitEvent(s, p->stream_switch, 0);
  if (e != hipSuccess) return hip_fail(p, e, "hipStreamWaitEvent(stream switch)");
  return GEMM_OK;
}

// Synchronise the last run's stream, read the sticky device status and clear it.
gemm_status take_device_status(gemm_plan *p) {
  if (!p->has_run) return GEMM_OK;
  hipError_t e = hipStreamSynchronize(p->last_stream);
  if (e != hipSuccess) return hip_fail(p, e, "hipStreamSynchronize");
  uint32_t st = 0;
  e = hipMemcpy(&st, p->d_status, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(p, e, "hipMemcpy(status)");
  if (st == 0) return GEMM_OK;
  const uint32_t zero = 0;
  e = hipMemcpy(p->d_status, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(p, e, "hipMemcpy(status clear)");
  p->last_error = "device-side scheduler error flags " + std::to_string(st) +
                  ((st & 1u) ? " (a workgroup gave up waiting at the concurrency gate and computed nothing)" : "") +
                  ((st & 2u) ? " (a claim-ring record answered the wrong ordinal)" : "");
  return (st & 2u) ? GEMM_E_SCHED : GEMM_E_TIMEOUT;
}

unsigned char *ctrl_set(gemm_plan *p, uint64_t run) { return p->d_ctrl_block + (run & 1u) * p->ctrl_set_bytes; }
// The set of launches captured into a graph: never cleared by another run, so
// those launches clean it up themselves (self_clean) for the next replay.
unsigned char *graph_set(gemm_plan *p) { return p->d_ctrl_block + 2 * p->ctrl_set_bytes; }
constexpr size_t kArrivalsOffset = sizeof(SchedCtrl);
constexpr size_t kVisitsOffset = sizeof(SchedCtrl) + sizeof(uint32_t) * (size_t)ptg::kMaxSplitTiles;

// K order of the default plan (see gemm_tile_desc.k_rotation).
constexpr int32_t kDefaultKRotation = GEMM_KROT_AUTO;

// The kernel's K order for a launch (0 = none, 1 = a phase per XCD region,
// 2 = two phases per region, 3 = a phase per key) from the plan's k_rotation.
// The phase follows the item id in a single GEMM and the problem in a grouped
// run. Only A's reads camp on shared low address bits (a k-step reads one
// column of every row of the tile's A panel, and every CU is at about the same
// k-step); B's reads of different tiles fall on different columns anyway. For a
// single GEMM the automatic choice therefore follows how many distinct A panels
// one XCD reads at once. Workgroup w runs on XCD w mod 8, so with at most 8
// tile columns an XCD's 32 concurrent tiles have 32 distinct A panels (every
// column of one panel row lands on a different XCD): two phases per region
// split them in halves that read different columns, at the price of reading
// the (shared) B panel slices at two phases. With more tile columns an XCD's
// tiles share A panels; one phase per region keeps them in step and still
// spreads the eight XCDs over K. A grouped run gets a phase per problem: a
// problem's tiles, which share its panels, walk K together, and the problems
// an XCD runs at once read different columns.
int32_t resolve_k_rotation(int32_t desc_value, bool grouped, int64_t N, int64_t bn) {
  switch (desc_value) {
    case GEMM_KROT_OFF: return 0;
    case GEMM_KROT_XCD: return 1;
    case GEMM_KROT_XCD2: return 2;
    case GEMM_KROT_UNIT: return 3;
    default: break;
  }
  if (grouped) return 3;
  if (N <= 0) return 0;
  return ceil_div(N, bn) <= 8 ? 2 : 1;
}

// Polls of the concurrency gate before a workgroup gives up (each well under a
// microsecond: a few seconds at most).
constexpr uint32_t kDefaultGateSpinLimit = 1u << 22;

// Fewest k-steps (of bk = 32) a K-chunk of a split tile gets.
constexpr int64_t kMinChunkSteps = 8;

// Chunk count of tail_split = GEMM_TAIL_SPLIT_AUTO for r split tiles of nk
// k-steps on `cus` compute units: the largest power of two up to 8 such that
// every chunk has an idle CU of its own (r S <= cus) and at least min_steps
// k-steps. A chunk's partial sum costs its tile a fix-up (one workgroup reads
// the S partials and writes the tile, 20-35 us for a 256 x 256 tile split four
// ways when 32-64 tiles fix up at once), so chunks must be long when many
// tiles split at once (64 k-steps from 32 split tiles on) and may be short
// when few do (16); 128 x 128 tiles carry a quarter of the work per k-step,
// so their chunks need four times the steps. Chosen from measurements on
// MI355X (256 x 256 tiles, dynamic, us, whole -> split): 2048^2 x 8192 (64
// tiles) 140 -> 98 at S = 4; 2048^2 x 4096 78 -> 64 at S = 2; 2048^2 x 2048
// 48, no split; 512^2 x 16384 (4 tiles) 255 -> 70 at S = 8; 257 tiles of
// 256 x 256 x 4096 205 -> 168 at S = 4 or 8.
int64_t auto_split_chunks(int64_t r, int64_t nk, int64_t cus, int32_t tile_edge) {
  if (r <= 0) return 1;
  const int64_t min_steps = (r >= 32 ? 64 : 16) * (tile_edge == 128 ? 4 : 1);
  const int64_t bound = std::min<int64_t>({8, cus / r, nk / min_steps});
  int64_t S = 1;
  while (S * 2 <= bound) S *= 2;
  return S;
}

// Work items of a run: T whole tiles, or, with tail splitting on, the tiles
// that fill whole waves of `workers` plus the r = T mod workers tiles of the
// partial last wave, each split into S K-chunks (S <= tail_split, <= workers / r
// so the chunks fit the idle workers, and >= kMinChunkSteps k-steps each). A
// run with fewer tiles than workers is one partial wave: all its tiles split.
// Work units (what one claim, static step or non-persistent block takes) are
// the items, or with claim groups g consecutive tiles (nothing is then split).
void plan_units(const gemm_plan *p, bool grouped, int32_t mode, int64_t tiles, int64_t K, int64_t *items,
                int64_t *split_base, int32_t *chunks, int32_t *group) {
  *items = tiles;
  *split_base = tiles;
  *chunks = 1;
  *group = 1;
  if (!grouped && p->desc.claim_group > 1) {
    *group = p->desc.claim_group;
    return;
  }
  const bool auto_split = p->desc.tail_split == GEMM_TAIL_SPLIT_AUTO;
  if (grouped || (!auto_split && p->desc.tail_split < 2) || p->ws_tiles == 0) return;
  const int64_t workers =
      mode == GEMM_SCHED_STATIC ? (int64_t)p->static_workers : (int64_t)p->occupancy * p->cu_count;
  if (workers < 2) return;
  const int64_t r = tiles % workers;
  if (r == 0 || r > ptg::kMaxSplitTiles) return;
  const int64_t nk = ceil_div(K, p->desc.bk);
  const int64_t S =
      auto_split ? std::min<int64_t>(auto_split_chunks(r, nk, std::max<int64_t>(1, workers / p->occupancy), p->desc.bm),
                                     p->ws_tiles / r)
                 : std::min<int64_t>({(int64_t)p->desc.tail_split, workers / r, nk / kMinChunkSteps, p->ws_tiles / r});
  if (S < 2) return;
  *split_base = tiles - r;
  *chunks = (int32_t)S;
  *items = tiles - r + r * S;
}

gemm_status launch(gemm_plan *p, int32_t mode, bool grouped, KernelArgs &args, int64_t tiles, int64_t K,
                   hipStream_t s) {
  if (mode < GEMM_SCHED_NONPERSISTENT || mode > GEMM_SCHED_DYNAMIC) return GEMM_E_INVALID_ARG;
  int64_t items = tiles, split_base = tiles;
  int32_t chunks = 1, group = 1;
  plan_units(p, grouped, mode, tiles, K, &items, &split_base, &chunks, &group);
  if (items > GEMM_MAX_TILES) return GEMM_E_SHAPE;
  const int64_t units = ceil_div(items, group);
  // Non-persistent: one workgroup per unit. Static: P workers. Dynamic: one
  // launch slot per unit, or (GEMM_GRID_RESIDENT) only the workgroups that can
  // be resident at once.
  int64_t grid = units;
  if (mode == GEMM_SCHED_STATIC) grid = std::min<int64_t>(units, p->static_workers);
  if (mode == GEMM_SCHED_DYNAMIC && p->desc.dynamic_grid == GEMM_GRID_RESIDENT)
    grid = std::min<int64_t>(units, (int64_t)p->occupancy * p->cu_count);
  args.T = (int32_t)units;
  args.first_wave = (int32_t)std::min<int64_t>(grid, (int64_t)p->occupancy * p->cu_count);
  args.items = (int32_t)items;
  args.claim_group = group;
  args.split_base = (int32_t)split_base;
  args.split_chunks = chunks;
  args.ws = p->d_ws;
  args.P = (int32_t)grid;
  args.claims_ahead = p->desc.claims_ahead;
  args.ring_depth = p->desc.ring_depth;
  args.claim_lead = p->desc.claim_lead;
  args.claim_policy = p->desc.claim_policy;
  args.raster_group = p->desc.raster == 1 ? p->desc.raster_group : 1;
  args.k_rotation = resolve_k_rotation(p->desc.k_rotation, grouped, args.single.N, p->desc.bn);
  args.counter_base = 0;
  if (mode == GEMM_SCHED_DYNAMIC && p->preset_pending) {
    args.counter_base = p->preset;
    p->preset_pending = false;
  }
  args.max_concurrent = p->desc.max_concurrent;
  args.gate_spin_limit = p->desc.gate_spin_limit > 0 ? (uint32_t)p->desc.gate_spin_limit : kDefaultGateSpinLimit;
  args.gate_base = 0;
  if (p->gate_preset_pending) {
    args.gate_base = p->gate_preset;
    p->gate_preset_pending = false;
  }
  args.status = p->d_status;
  args.log_cap = p->desc.log_capacity;
  // An uncaptured run uses set runs % 2 and clears the other for the next run;
  // a launch being captured into a graph uses the graph set, clears nothing
  // and leaves its set at zero itself, so that every replay starts clean.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &capture);
  if (e != hipSuccess) return hip_fail(p, e, "hipStreamIsCapturing");
  const bool captured = capture != hipStreamCaptureStatusNone;
  unsigned char *cur = captured ? graph_set(p) : ctrl_set(p, p->runs);
  args.ctrl = reinterpret_cast<SchedCtrl *>(cur);
  args.arrivals = reinterpret_cast<uint32_t *>(cur + kArrivalsOffset);
  args.visits = reinterpret_cast<uint32_t *>(cur + kVisitsOffset);
  if (captured) {
    args.ctrl_next = nullptr;
    args.clear_next = nullptr;
    args.clear_count = 0;
    args.self_clean = 1;
  } else {
    unsigned char *nxt = ctrl_set(p, p->runs + 1);
    args.ctrl_next = reinterpret_cast<SchedCtrl *>(nxt);
    args.clear_next = reinterpret_cast<uint32_t *>(nxt + kArrivalsOffset);
    args.clear_count = ptg::kMaxSplitTiles + p->desc.log_capacity;
    args.self_clean = 0;
  }
  args.log = p->d_log;
  e = ptg::launch_gemm(p->desc.bm, mode, grouped, p->desc.b_layout == 1, args, (int)grid, p->dyn_lds, s);
  if (e != hipSuccess) return hip_fail(p, e, "kernel launch");
  if (!captured) ++p->runs;
  p->last_set = cur;
  p->last_stream = s;
  p->has_run = true;
  p->last_tiles = tiles;
  p->last_units = units;
  p->last_items = items;
  p->last_split_base = split_base;
  p->last_split_chunks = chunks;
  p->last_claim_group = group;
  p->last_grid = grid;
  p->last_mode = mode;
  p->last_k_rotation = GEMM_KROT_OFF + args.k_rotation;  // kernel order 0..3 -> GEMM_KROT_OFF.._UNIT
  return GEMM_OK;
}

// ---- scratch of gemm_run_noalloc: the scheduler state in a file-scope device
// array (each device holds its own copy until the process ends), so the entry
// point never allocates. Layout: two control sets of 4352 bytes (the control
// block: claim counters, gate, error word and the exit groups; run i uses set
// i % 2 and clears the other for run i + 1, as a plan's sets do), then a
// 256-byte status word block: 8960 bytes. The configuration is fixed (no log,
// no split tail, no gate), so nothing in it grows with the problem.
constexpr size_t kNoallocSetBytes = (sizeof(SchedCtrl) + 255) & ~(size_t)255;
constexpr size_t kNoallocScratchBytes = 2 * kNoallocSetBytes + 256;
static_assert(sizeof(SchedCtrl) <= kNoallocSetBytes && kNoallocScratchBytes == 8960, "control set");
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

__global__ void ptg_zero_words(uint32_t *p, uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

struct NoallocDevice {
  bool ready = false;
  unsigned char *ptr = nullptr;  // device address of `scratch` on this device
  int cu_count = 0;
  int occupancy = 0;
  uint64_t runs = 0;
};
constexpr int kNoallocMaxDevices = 64;
NoallocDevice g_noalloc[kNoallocMaxDevices];
std::mutex g_noalloc_mutex;

// Once per device, with that device current: check it, resolve the device
// address of `scratch` (the array's name is only a host-side stand-in) and
// clear the array with a fill kernel on `s` (not a memset, so a caller that
// captures the first call into a graph records a kernel node).
gemm_status noalloc_setup(int dev, hipStream_t s, NoallocDevice **out) {
  NoallocDevice &d = g_noalloc[dev];
  if (d.ready) {
    *out = &d;
    return GEMM_OK;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_E_UNSUPPORTED;
  void *ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GEMM_E_HIP;
  int occ = 0;
  if (ptg::gemm_occupancy(256, 0, &occ) != hipSuccess || occ < 1) return GEMM_E_HIP;
  hipLaunchKernelGGL(ptg_zero_words, dim3(1), dim3(64), 0, s, static_cast<uint32_t *>(ptr),
                     (uint32_t)(kNoallocScratchBytes / sizeof(uint32_t)));
  if (hipGetLastError() != hipSuccess) return GEMM_E_HIP;
  d.ptr = static_cast<unsigned char *>(ptr);
  d.cu_count = prop.multiProcessorCount;
  d.occupancy = occ;
  d.runs = 0;
  d.ready = true;
  *out = &d;
  return GEMM_OK;
}

}  // namespace

extern "C" {

const char *gemm_status_str(int32_t status) {
  switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_E_INVALID_ARG: return "invalid argument";
    case GEMM_E_SHAPE: return "unsupported shape (negative, K or N not a multiple of 8, or over a size limit)";
    case GEMM_E_UNSUPPORTED: return "unsupported device or tile configuration (gfx950 only; tiles 128x128x32 or 256x256x32)";
    case GEMM_E_DEVICE: return "plan used while a different device is current";
    case GEMM_E_HIP: return "HIP runtime error";
    case GEMM_E_NOMEM: return "out of memory";
    case GEMM_E_TIMEOUT: return "timed out waiting";
    case GEMM_E_SCHED: return "device-side claim-ring protocol violation";
    default: return "unknown status";
  }
}

gemm_status gemm_default_desc(gemm_tile_desc *out, int32_t tile_edge, int32_t device) {
  if (!out) return GEMM_E_INVALID_ARG;
  if (tile_edge != 128 && tile_edge != 256) return GEMM_E_UNSUPPORTED;
  std::memset(out, 0, sizeof(*out));
  out->bm = out->bn = tile_edge;
  out->bk = 32;
  out->ring_depth = 3;
  out->claims_ahead = 1;
  out->claim_lead = 4;
  out->claim_policy = 1;
  out->raster = 0;
  out->raster_group = 8;
  out->static_workers = 0;
  out->log_capacity = 0;
  out->min_lds_bytes = 0;
  out->max_concurrent = 0;
  out->max_groups = 1024;
  out->device = device;
  out->tail_split = 0;
  out->group_order = 0;
  out->claim_group = 1;
  out->b_layout = 0;
  out->gate_spin_limit = 0;
  out->k_rotation = kDefaultKRotation;
  out->dynamic_grid = GEMM_GRID_ALL;
  return GEMM_OK;
}

gemm_status gemm_create(gemm_tile_cfg *out, const gemm_tile_desc *desc) {
  if (!out || !desc) return GEMM_E_INVALID_ARG;
  *out = nullptr;
  const gemm_tile_desc d = *desc;
  if (!valid_tile(d)) return GEMM_E_UNSUPPORTED;
  if (d.ring_depth < 2 || d.ring_depth > 3) return GEMM_E_INVALID_ARG;
  if (d.claims_ahead < 0 || d.claims_ahead > 2 || d.claims_ahead >= d.ring_depth) return GEMM_E_INVALID_ARG;
  if (d.claim_lead < 0 || d.claim_policy < 0 || d.claim_policy > 2) return GEMM_E_INVALID_ARG;
  if (d.raster < 0 || d.raster > 1 || (d.raster == 1 && d.raster_group < 1)) return GEMM_E_INVALID_ARG;
  if (d.static_workers < 0 || d.log_capacity < 0 || d.min_lds_bytes < 0 || d.max_concurrent < 0 ||
      d.max_groups < 0 || d.tail_split < GEMM_TAIL_SPLIT_AUTO || d.tail_split > GEMM_MAX_TAIL_SPLIT || d.group_order < 0 ||
      d.group_order > 1 || d.claim_group < 0 || d.claim_group > GEMM_MAX_CLAIM_GROUP || d.b_layout < 0 ||
      d.b_layout > 1 || d.gate_spin_limit < 0 || d.k_rotation < GEMM_KROT_AUTO || d.k_rotation > GEMM_KROT_UNIT ||
      d.dynamic_grid < GEMM_GRID_ALL || d.dynamic_grid > GEMM_GRID_RESIDENT)
    return GEMM_E_INVALID_ARG;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return GEMM_E_HIP;
  if (d.device < 0 || d.device >= ndev) return GEMM_E_INVALID_ARG;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, d.device);
  if (e != hipSuccess) return GEMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_E_UNSUPPORTED;
  int cur = 0;
  e = hipGetDevice(&cur);
  if (e != hipSuccess) return GEMM_E_HIP;
  if (cur != d.device) return GEMM_E_DEVICE;

  gemm_plan *p = new (std::nothrow) gemm_plan();
  if (!p) return GEMM_E_NOMEM;
  p->desc = d;
  if (p->desc.max_groups == 0) p->desc.max_groups = 1024;
  p->cu_count = prop.multiProcessorCount;
  int wclk = 0;
  if (hipDeviceGetAttribute(&wclk, hipDeviceAttributeWallClockRate, d.device) == hipSuccess) p->wallclock_khz = wclk;
  const int static_lds = ptg::gemm_static_lds_bytes(d.bm);
  p->dyn_lds = 0;
  if (d.min_lds_bytes > static_lds) p->dyn_lds = d.min_lds_bytes - static_lds;
  p->lds_bytes = static_lds + p->dyn_lds;
  if (p->lds_bytes > (int)prop.sharedMemPerBlock) {
    delete p;
    return GEMM_E_INVALID_ARG;
  }
  int occ = 0;
  e = ptg::gemm_occupancy(d.bm, p->dyn_lds, &occ);
  if (e != hipSuccess || occ < 1) {
    delete p;
    return GEMM_E_HIP;
  }
  p->occupancy = occ;
  p->static_workers = d.static_workers > 0 ? d.static_workers : occ * p->cu_count;

  p->ctrl_set_bytes = (kVisitsOffset + sizeof(uint32_t) * (size_t)std::max(d.log_capacity, 1) + 255) & ~(size_t)255;
  if (hipMalloc(&p->d_ctrl_block, 3 * p->ctrl_set_bytes + 256) != hipSuccess) {
    delete p;
    return GEMM_E_NOMEM;
  }
  p->d_status = reinterpret_cast<uint32_t *>(p->d_ctrl_block + 3 * p->ctrl_set_bytes);
  if (hipMemset(p->d_ctrl_block, 0, 3 * p->ctrl_set_bytes + 256) != hipSuccess) {
    gemm_destroy(p);
    return GEMM_E_HIP;
  }
  if (d.log_capacity > 0) {
    if (hipMalloc(&p->d_log, sizeof(TileRecDev) * (size_t)d.log_capacity) != hipSuccess) {
      gemm_destroy(p);
      return GEMM_E_NOMEM;
    }
  }
  if (d.tail_split >= 2 || d.tail_split == GEMM_TAIL_SPLIT_AUTO) {
    // the K-chunks of one run never outnumber the workers of one wave
    p->ws_tiles = std::max<int64_t>((int64_t)occ * p->cu_count, p->static_workers);
    if (hipMalloc(&p->d_ws, sizeof(float) * (size_t)d.bm * (size_t)d.bn * (size_t)p->ws_tiles) != hipSuccess) {
      p->d_ws = nullptr;
      p->ws_tiles = 0;
      gemm_destroy(p);
      return GEMM_E_NOMEM;
    }
  }
  if (hipMalloc(&p->d_groups, sizeof(KernelProblem) * (size_t)p->desc.max_groups) != hipSuccess) {
    gemm_destroy(p);
    return GEMM_E_NOMEM;
  }
  if (hipHostMalloc(&p->h_groups, sizeof(KernelProblem) * (size_t)p->desc.max_groups, hipHostMallocDefault) !=
      hipSuccess) {
    p->h_groups = nullptr;
    gemm_destroy(p);
    return GEMM_E_NOMEM;
  }
  if (hipEventCreateWithFlags(&p->groups_uploaded, hipEventDisableTiming) != hipSuccess) {
    p->groups_uploaded = nullptr;
    gemm_destroy(p);
    return GEMM_E_HIP;
  }
  if (hipEventCreateWithFlags(&p->stream_switch, hipEventDisableTiming) != hipSuccess) {
    p->stream_switch = nullptr;
    gemm_destroy(p);
    return GEMM_E_HIP;
  }
  *out = p;
  return GEMM_OK;
}

gemm_status gemm_run(const void *A, const void *B, float *C, int64_t M, int64_t N, int64_t K, int32_t sched_mode,
                     gemm_tile_cfg tile_cfg, void *stream) {
  gemm_plan *p = tile_cfg;
  if (!p) return GEMM_E_INVALID_ARG;
  if (sched_mode < GEMM_SCHED_NONPERSISTENT || sched_mode > GEMM_SCHED_DYNAMIC) return GEMM_E_INVALID_ARG;
  gemm_status st = check_problem(A, B, C, M, N, K);
  if (st != GEMM_OK) return st;
  st = check_current_device(p);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  const int64_t tm = ceil_div(M, p->desc.bm), tn = ceil_div(N, p->desc.bn);
  const int64_t tiles = tm * tn;
  if (tiles > GEMM_MAX_TILES) return GEMM_E_SHAPE;
  KernelArgs args;
  std::memset(&args, 0, sizeof(args));
  args.single.A = static_cast<const uint16_t *>(A);
  args.single.B = static_cast<const uint16_t *>(B);
  args.single.C = C;
  args.single.M = (int32_t)M;
  args.single.N = (int32_t)N;
  args.single.K = (int32_t)K;
  args.single.tiles_m = (int32_t)tm;
  args.single.tiles_n = (int32_t)tn;
  args.single.tile_start = 0;
  args.single.unit_start = 0;
  args.groups = nullptr;
  args.G = 1;
  st = order_after_last_stream(p, static_cast<hipStream_t>(stream));
  if (st != GEMM_OK) return st;
  p->last_tile_start.assign(1, 0);
  p->last_k.assign(1, (int32_t)K);
  p->last_unit_map.clear();
  return launch(p, sched_mode, false, args, tiles, K, static_cast<hipStream_t>(stream));
}

gemm_status gemm_run_noalloc(const void *A, const void *B, float *C, int64_t M, int64_t N, int64_t K,
                             int32_t sched_mode, uint32_t *d_status, void *stream) {
  if (sched_mode < GEMM_SCHED_NONPERSISTENT || sched_mode > GEMM_SCHED_DYNAMIC) return GEMM_E_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(d_status) & 3u) != 0) return GEMM_E_INVALID_ARG;
  gemm_status st = check_problem(A, B, C, M, N, K);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  const int64_t tm = ceil_div(M, 256), tn = ceil_div(N, 256);
  const int64_t tiles = tm * tn;
  if (tiles > GEMM_MAX_TILES) return GEMM_E_SHAPE;  // the scratch does not grow with the problem
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_E_HIP;
  if (dev < 0 || dev >= kNoallocMaxDevices) return GEMM_E_DEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_noalloc_mutex);
  NoallocDevice *d = nullptr;
  st = noalloc_setup(dev, s, &d);
  if (st != GEMM_OK) return st;
  KernelArgs args;
  std::memset(&args, 0, sizeof(args));
  args.single.A = static_cast<const uint16_t *>(A);
  args.single.B = static_cast<const uint16_t *>(B);
  args.single.C = C;
  args.single.M = (int32_t)M;
  args.single.N = (int32_t)N;
  args.single.K = (int32_t)K;
  args.single.tiles_m = (int32_t)tm;
  args.single.tiles_n = (int32_t)tn;
  args.G = 1;
  // the default plan's configuration (gemm_default_desc with tile edge 256)
  const int64_t workers = (int64_t)d->occupancy * d->cu_count;
  const int64_t grid = sched_mode == GEMM_SCHED_STATIC ? std::min<int64_t>(tiles, workers) : tiles;
  args.T = (int32_t)tiles;
  args.first_wave = (int32_t)std::min<int64_t>(grid, workers);
  args.items = (int32_t)tiles;
  args.claim_group = 1;
  args.split_base = (int32_t)tiles;
  args.split_chunks = 1;
  args.P = (int32_t)grid;
  args.claims_ahead = 1;
  args.ring_depth = 3;
  args.claim_lead = 4;
  args.claim_policy = 1;
  args.raster_group = 1;
  args.k_rotation = resolve_k_rotation(kDefaultKRotation, false, N, 256);
  args.gate_spin_limit = kDefaultGateSpinLimit;
  unsigned char *cur = d->ptr + (d->runs & 1u) * kNoallocSetBytes;
  unsigned char *nxt = d->ptr + ((d->runs + 1) & 1u) * kNoallocSetBytes;
  args.ctrl = reinterpret_cast<SchedCtrl *>(cur);
  // no split tail and no log: the arrival and visit counters are never touched;
  // they point at the unused rest of the set
  args.arrivals = reinterpret_cast<uint32_t *>(cur + sizeof(SchedCtrl));
  args.visits = reinterpret_cast<uint32_t *>(cur + sizeof(SchedCtrl));
  args.ctrl_next = reinterpret_cast<SchedCtrl *>(nxt);
  args.clear_next = nullptr;
  args.clear_count = 0;
  args.self_clean = 1;  // callers capture it into graphs: every run leaves its set at zero
  args.status = d_status ? d_status : reinterpret_cast<uint32_t *>(d->ptr + 2 * kNoallocSetBytes);
  hipError_t e = ptg::launch_gemm(256, sched_mode, false, false, args, (int)grid, 0, s);
  if (e != hipSuccess) return GEMM_E_HIP;
  ++d->runs;
  return GEMM_OK;
}

gemm_status gemm_run_grouped(int32_t G, const void *const *A, const void *const *B, float *const *C,
                             const int64_t *M, const int64_t *N, const int64_t *K, int32_t sched_mode,
                             gemm_tile_cfg tile_cfg, void *stream) {
  gemm_plan *p = tile_cfg;
  if (!p) return GEMM_E_INVALID_ARG;
  if (G <= 0 || !A || !B || !C || !M || !N || !K) return GEMM_E_INVALID_ARG;
  if (G > p->desc.max_groups) return GEMM_E_SHAPE;
  if (sched_mode < GEMM_SCHED_NONPERSISTENT || sched_mode > GEMM_SCHED_DYNAMIC) return GEMM_E_INVALID_ARG;
  std::vector<KernelProblem> probs((size_t)G);
  std::vector<int32_t> starts((size_t)G), ks((size_t)G);
  int64_t tiles = 0;
  for (int32_t g = 0; g < G; ++g) {
    gemm_status st = check_problem(A[g], B[g], C[g], M[g], N[g], K[g]);
    if (st != GEMM_OK) return st;
    KernelProblem &q = probs[(size_t)g];
    q.A = static_cast<const uint16_t *>(A[g]);
    q.B = static_cast<const uint16_t *>(B[g]);
    q.C = C[g];
    q.M = (int32_t)M[g];
    q.N = (int32_t)N[g];
    q.K = (int32_t)K[g];
    q.tiles_m = (int32_t)ceil_div(M[g], p->desc.bm);
    q.tiles_n = (int32_t)ceil_div(N[g], p->desc.bn);
    q.tile_start = (int32_t)tiles;
    q.unit_start = (int32_t)tiles;
    starts[(size_t)g] = (int32_t)tiles;
    ks[(size_t)g] = (int32_t)K[g];
    tiles += (int64_t)q.tiles_m * q.tiles_n;
    if (tiles > GEMM_MAX_TILES) return GEMM_E_SHAPE;
  }
  gemm_status st = check_current_device(p);
  if (st != GEMM_OK) return st;
  if (tiles == 0) return GEMM_OK;
  // claim order: problems as given, or longest K first (every tile of a problem
  // costs about K; handing out the costly tiles first keeps the short ones for
  // the end, where they fill the gaps: longest-processing-time order). The table
  // goes to the device in claim order; tile ids keep the call-order numbering.
  // With contiguous XCD regions (claim policy 2) each region is one run of the
  // claim order, so the sorted problems are dealt to the eight runs in snake
  // order (0..7, 7..0, ...): every region starts with its share of the longest
  // problems and the regions' totals stay close.
  std::vector<KernelProblem> table = probs;
  if (p->desc.group_order == 1) {
    std::stable_sort(table.begin(), table.end(),
                     [](const KernelProblem &a, const KernelProblem &b) { return a.K > b.K; });
    if (p->desc.claim_policy == 2) {
      std::vector<KernelProblem> dealt[ptg::kXcdRegions];
      for (size_t i = 0; i < table.size(); ++i) {
        const size_t round = i / ptg::kXcdRegions, pos = i % ptg::kXcdRegions;
        dealt[round % 2 == 0 ? pos : ptg::kXcdRegions - 1 - pos].push_back(table[i]);
      }
      table.clear();
      for (const auto &d : dealt) table.insert(table.end(), d.begin(), d.end());
    }
    int32_t u = 0;
    for (KernelProblem &q : table) {
      q.unit_start = u;
      u += q.tiles_m * q.tiles_n;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = order_after_last_stream(p, s);
  if (st != GEMM_OK) return st;
  const bool same = p->last_groups.size() == table.size() &&
                    std::memcmp(p->last_groups.data(), table.data(), sizeof(KernelProblem) * table.size()) == 0;
  if (!same) {
    // the pinned staging may still be the source of an earlier upload
    if (p->groups_event_pending) {
      hipError_t e = hipEventSynchronize(p->groups_uploaded);
      if (e != hipSuccess) return hip_fail(p, e, "hipEventSynchronize(groups)");
    }
    std::memcpy(p->h_groups, table.data(), sizeof(KernelProblem) * table.size());
    hipError_t e = hipMemcpyAsync(p->d_groups, p->h_groups, sizeof(KernelProblem) * table.size(),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(p, e, "hipMemcpyAsync(groups)");
    e = hipEventRecord(p->groups_uploaded, s);
    if (e != hipSuccess) return hip_fail(p, e, "hipEventRecord(groups)");
    p->groups_event_pending = true;
    p->last_groups = table;
  }
  KernelArgs args;
  std::memset(&args, 0, sizeof(args));
  args.single = table[0];
  args.groups = p->d_groups;
  args.G = G;
  p->last_tile_start = starts;
  p->last_k = ks;
  p->last_unit_map.clear();
  for (const KernelProblem &q : table) p->last_unit_map.emplace_back(q.unit_start, q.tile_start);
  return launch(p, sched_mode, true, args, tiles, 0, s);
}

gemm_status gemm_read_log(gemm_tile_cfg tile_cfg, gemm_tile_rec *host_out, size_t cap, size_t *n_out) {
  gemm_plan *p = tile_cfg;
  if (!p || !n_out || (cap > 0 && !host_out)) return GEMM_E_INVALID_ARG;
  *n_out = 0;
  if (!p->has_run) return GEMM_OK;
  // the device status first (it also synchronises the stream): it is reported
  // whether or not the log is on
  const gemm_status dev_status = take_device_status(p);
  if (dev_status == GEMM_E_HIP) return dev_status;
  if (p->desc.log_capacity == 0) return dev_status;
  hipError_t e = hipSuccess;
  const size_t n = (size_t)std::min<int64_t>(p->last_items, p->desc.log_capacity);
  const size_t m = std::min(n, cap);
  std::vector<TileRecDev> recs(m);
  std::vector<uint32_t> visits(m);
  if (m > 0) {
    e = hipMemcpy(recs.data(), p->d_log, sizeof(TileRecDev) * m, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(p, e, "hipMemcpy(log)");
    e = hipMemcpy(visits.data(), p->last_set + kVisitsOffset, sizeof(uint32_t) * m,
                  hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(p, e, "hipMemcpy(visits)");
  }
  const int64_t bk = p->desc.bk;
  for (size_t i = 0; i < m; ++i) {
    gemm_tile_rec &r = host_out[i];
    std::memset(&r, 0, sizeof(r));
    r.visits = visits[i];
    // the item's tile, K range and unit as the launch planned them
    int64_t tile = (int64_t)i, chunk = 0;
    const int64_t S = p->last_split_chunks;
    r.unit = (uint32_t)((int64_t)i / p->last_claim_group);
    if ((int64_t)i >= p->last_split_base) {
      tile = p->last_split_base + ((int64_t)i - p->last_split_base) / S;
      chunk = ((int64_t)i - p->last_split_base) % S;
    } else if (!p->last_unit_map.empty()) {
      const auto &um = p->last_unit_map;
      const auto it = std::upper_bound(um.begin(), um.end(), std::make_pair((int32_t)i, INT32_MAX));
      const auto &e0 = *(it - 1);
      tile = e0.second + ((int64_t)i - e0.first);
    }
    const auto &ts = p->last_tile_start;
    const size_t g = (size_t)(std::upper_bound(ts.begin(), ts.end(), (int32_t)tile) - ts.begin() - 1);
    const int64_t Kg = p->last_k.empty() ? 0 : p->last_k[g];
    const int64_t nk = ceil_div(Kg, bk);
    const int64_t kb = (int64_t)i >= p->last_split_base ? nk * chunk / S : 0;
    const int64_t ke = (int64_t)i >= p->last_split_base ? nk * (chunk + 1) / S : nk;
    r.problem = (uint32_t)g;
    if (visits[i] == 0) {
      r.tile = (uint32_t)tile;
      r.k_begin = (uint32_t)std::min(kb * bk, Kg);
      r.k_end = (uint32_t)std::min(ke * bk, Kg);
      r.worker = 0xFFFFFFFFu;
      continue;
    }
    // what the kernel recorded (the tests compare it with the plan above)
    r.k_begin = (uint32_t)std::min((int64_t)recs[i].kb * bk, Kg);
    r.k_end = (uint32_t)std::min((int64_t)recs[i].ke * bk, Kg);
    r.tile = recs[i].tile;
    r.unit = recs[i].unit;
    r.worker = recs[i].worker;
    r.hw_id = recs[i].hw_id;
    r.xcc_id = recs[i].xcc_id;
    r.t0 = recs[i].t0;
    r.t1 = recs[i].t1;
    r.r0 = recs[i].r0;
    r.r1 = recs[i].r1;
  }
  *n_out = m;
  return dev_status;
}

gemm_status gemm_sync(gemm_tile_cfg tile_cfg) {
  gemm_plan *p = tile_cfg;
  if (!p) return GEMM_E_INVALID_ARG;
  return take_device_status(p);
}

gemm_status gemm_plan_info_get(gemm_tile_cfg tile_cfg, gemm_plan_info *out) {
  gemm_plan *p = tile_cfg;
  if (!p || !out) return GEMM_E_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  out->device = p->desc.device;
  out->cu_count = p->cu_count;
  out->occupancy = p->occupancy;
  out->static_workers = p->static_workers;
  out->wallclock_khz = p->wallclock_khz;
  out->last_tiles = p->last_tiles;
  out->last_units = p->last_units;
  out->last_items = p->last_items;
  out->last_split_base = p->last_split_base;
  out->last_split_chunks = p->last_split_chunks;
  out->last_claim_group = p->last_claim_group;
  out->last_grid = p->last_grid;
  out->last_mode = p->last_mode;
  out->lds_bytes = p->lds_bytes;
  out->last_k_rotation = p->last_k_rotation;
  return GEMM_OK;
}

gemm_status gemm_destroy(gemm_tile_cfg tile_cfg) {
  gemm_plan *p = tile_cfg;
  if (!p) return GEMM_OK;
  if (p->has_run) (void)hipStreamSynchronize(p->last_stream);
  if (p->groups_event_pending && p->groups_uploaded) (void)hipEventSynchronize(p->groups_uploaded);
  if (p->d_ctrl_block) (void)hipFree(p->d_ctrl_block);
  if (p->d_log) (void)hipFree(p->d_log);
  if (p->d_ws) (void)hipFree(p->d_ws);
  if (p->d_groups) (void)hipFree(p->d_groups);
  if (p->h_groups) (void)hipHostFree(p->h_groups);
  if (p->groups_uploaded) (void)hipEventDestroy(p->groups_uploaded);
  if (p->stream_switch) (void)hipEventDestroy(p->stream_switch);
  delete p;
  return GEMM_OK;
}

const char *gemm_last_hip_error(gemm_tile_cfg tile_cfg) {
  if (!tile_cfg) return "";
  return tile_cfg->last_error.c_str();
}

gemm_status gemm_test_preset_counter(gemm_tile_cfg tile_cfg, uint32_t start) {
  gemm_plan *p = tile_cfg;
  if (!p) return GEMM_E_INVALID_ARG;
  p->preset = start;
  p->preset_pending = true;
  return GEMM_OK;
}

gemm_status gemm_test_preset_gate(gemm_tile_cfg tile_cfg, uint32_t held) {
  gemm_plan *p = tile_cfg;
  if (!p) return GEMM_E_INVALID_ARG;
  p->gate_preset = held;
  p->gate_preset_pending = true;
  return GEMM_OK;
}

gemm_status gemm_test_stream_cu_mask(void **out_stream, int32_t device, const uint32_t *mask, uint32_t words) {
  if (!out_stream || !mask || words == 0 || words > 64) return GEMM_E_INVALID_ARG;
  *out_stream = nullptr;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_E_HIP;
  if (cur != device) return GEMM_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return GEMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_E_UNSUPPORTED;
  // every compute unit the mask names must exist, and at least one must be named
  uint32_t named = 0;
  for (uint32_t w = 0; w < words; ++w) {
    for (uint32_t b = 0; b < 32; ++b) {
      if (!((mask[w] >> b) & 1u)) continue;
      if ((int64_t)w * 32 + b >= prop.multiProcessorCount) return GEMM_E_INVALID_ARG;
      ++named;
    }
  }
  if (named == 0) return GEMM_E_INVALID_ARG;
  hipStream_t s = nullptr;
  if (hipExtStreamCreateWithCUMask(&s, words, mask) != hipSuccess) return GEMM_E_HIP;
  *out_stream = s;
  return GEMM_OK;
}

gemm_status gemm_test_stream_destroy(void *stream) {
  if (!stream) return GEMM_E_INVALID_ARG;
  return hipStreamDestroy(static_cast<hipStream_t>(stream)) == hipSuccess ? GEMM_OK : GEMM_E_HIP;
}

gemm_status gemm_test_spoiler(int32_t device, int32_t n_wgs, int64_t spin_ns, void *stream, uint64_t *d_log,
                              double wait_resident_ms) {
  if (n_wgs <= 0 || spin_ns < 0 || spin_ns > 60ll * 1000 * 1000 * 1000) return GEMM_E_INVALID_ARG;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_E_HIP;
  if (cur != device) return GEMM_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return GEMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_E_UNSUPPORTED;
  if (n_wgs > prop.multiProcessorCount) return GEMM_E_INVALID_ARG;  // one workgroup per CU
  int wclk = 0;
  if (hipDeviceGetAttribute(&wclk, hipDeviceAttributeWallClockRate, device) != hipSuccess || wclk <= 0)
    return GEMM_E_HIP;
  // one host-visible residency counter per process (a device has its own launch order)
  static uint32_t *resident = nullptr;
  if (!resident) {
    if (hipHostMalloc(&resident, 64, hipHostMallocCoherent) != hipSuccess) {
      resident = nullptr;
      return GEMM_E_NOMEM;
    }
  }
  __atomic_store_n(resident, 0u, __ATOMIC_SEQ_CST);
  const uint64_t ticks = (uint64_t)((double)spin_ns * (double)wclk / 1.0e6);
  hipError_t e = ptg::launch_spoiler(n_wgs, ticks, resident, d_log, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return GEMM_E_HIP;
  if (wait_resident_ms > 0) {
    const auto t_end = std::chrono::steady_clock::now() + std::chrono::duration<double, std::milli>(wait_resident_ms);
    while (__atomic_load_n(resident, __ATOMIC_SEQ_CST) < (uint32_t)n_wgs) {
      if (std::chrono::steady_clock::now() > t_end) return GEMM_E_TIMEOUT;
      std::this_thread::yield();
    }
  }
  return GEMM_OK;
}

gemm_status gemm_mfma_probe(int32_t device, int32_t iters, int32_t random_operands, int32_t mfma_block,
                            double *tflops_out, double *clock_ghz_out) {
  if (!tflops_out || !clock_ghz_out || iters < 1 || iters > 10000000) return GEMM_E_INVALID_ARG;
  if (mfma_block != 16 && mfma_block != 32) return GEMM_E_INVALID_ARG;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_E_HIP;
  if (cur != device) return GEMM_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return GEMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_E_UNSUPPORTED;
  const int grid = prop.multiProcessorCount;
  float *sink = nullptr;
  uint64_t *ticks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  gemm_status st = GEMM_OK;
  std::vector<uint64_t> h((size_t)grid * 2);
  float ms = 0.0f;
  if (hipMalloc(&sink, sizeof(float) * 256 * (size_t)grid) != hipSuccess ||
      hipMalloc(&ticks, sizeof(uint64_t) * 2 * (size_t)grid) != hipSuccess) {
    st = GEMM_E_NOMEM;
  } else if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess ||
             hipEventRecord(e0, nullptr) != hipSuccess ||
             ptg::launch_mfma_probe(grid, iters, random_operands != 0, mfma_block, sink, ticks, nullptr) != hipSuccess ||
             hipEventRecord(e1, nullptr) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
             hipEventElapsedTime(&ms, e0, e1) != hipSuccess ||
             hipMemcpy(h.data(), ticks, sizeof(uint64_t) * h.size(), hipMemcpyDeviceToHost) != hipSuccess) {
    st = GEMM_E_HIP;
  }
  if (st == GEMM_OK) {
    int wclk = 0;
    if (hipDeviceGetAttribute(&wclk, hipDeviceAttributeWallClockRate, device) != hipSuccess || wclk <= 0) {
      st = GEMM_E_HIP;
    } else {
      double ratio = 0.0;
      for (int i = 0; i < grid; ++i) ratio += (double)h[2 * i] / (double)std::max<uint64_t>(h[2 * i + 1], 1);
      ratio /= grid;
      // 4 waves x (8 MFMAs of 32*32*16*2 or 16 of 16*16*32*2) flop per round and workgroup
      const double flops = 4.0 * 262144.0 * (double)iters * (double)grid;
      *tflops_out = flops / ((double)ms * 1e-3) / 1e12;
      *clock_ghz_out = ratio * (double)wclk * 1e-6;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (ticks) (void)hipFree(ticks);
  return st;
}

gemm_status gemm_hbm_probe(int32_t device, int64_t bytes, int32_t kind, int32_t reps, double *gbs_out) {
  if (!gbs_out || kind < 0 || kind > 1 || reps < 1 || reps > 1000) return GEMM_E_INVALID_ARG;
  if (bytes < (1 << 20) || bytes > (int64_t)16 << 30 || (bytes % 4096) != 0) return GEMM_E_INVALID_ARG;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GEMM_E_HIP;
  if (cur != device) return GEMM_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return GEMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_E_UNSUPPORTED;
  const int grid = 4 * prop.multiProcessorCount;
  void *src = nullptr, *dst = nullptr;
  float *sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  gemm_status st = GEMM_OK;
  float ms = 0.0f;
  if (hipMalloc(&src, (size_t)bytes) != hipSuccess || (kind == 1 && hipMalloc(&dst, (size_t)bytes) != hipSuccess) ||
      hipMalloc(&sink, sizeof(float) * (size_t)grid) != hipSuccess) {
    st = GEMM_E_NOMEM;
  } else if (hipMemset(src, 0, (size_t)bytes) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
             hipEventCreate(&e1) != hipSuccess) {
    st = GEMM_E_HIP;
  } else {
    bool ok = true;
    for (int w = 0; w < 3 && ok; ++w) ok = ptg::launch_hbm_probe(kind, grid, src, dst, (size_t)bytes, sink, nullptr) == hipSuccess;
    ok = ok && hipEventRecord(e0, nullptr) == hipSuccess;
    for (int r = 0; r < reps && ok; ++r)
      ok = ptg::launch_hbm_probe(kind, grid, src, dst, (size_t)bytes, sink, nullptr) == hipSuccess;
    ok = ok && hipEventRecord(e1, nullptr) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
         hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    if (!ok || ms <= 0.0f) st = GEMM_E_HIP;
  }
  if (st == GEMM_OK) {
    // bytes moved: read once (kind 0), or read and written (kind 1)
    const double moved = (double)bytes * (kind == 1 ? 2.0 : 1.0) * (double)reps;
    *gbs_out = moved / ((double)ms * 1e-3) / 1e9;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (src) (void)hipFree(src);
  if (dst) (void)hipFree(dst);
  if (sink) (void)hipFree(sink);
  return st;
}

}  // extern "C"

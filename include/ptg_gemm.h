/*
 * ptg_gemm.h - C ABI of the persistent tiled bf16 GEMM for MI355X (gfx950).
 *
 * Operation. C[m][n] = sum_k A[m][k] * B[k][n] with A, B in bf16 and C in fp32
 * (fp32 accumulation, C overwritten). The output is cut into BM x BN tiles;
 * each tile is one unit of work over the whole K extent, computed exactly once
 * by one worker (a workgroup). Sources: "CUTLASS Cluster Launch Control dynamic
 * persistent kernel" (blog post), section "from one tile per block to one
 * worker computing continuously" (a unit is one full output tile, no split-K)
 * and section "cancelling the launch, receiving the work coordinate" (each
 * unit has exactly one owner).
 *
 * Schedulers (same blog post, the three-mode table in the first section):
 *   GEMM_SCHED_NONPERSISTENT  grid = all tiles; block b computes tile b and exits.
 *   GEMM_SCHED_STATIC         grid = P workers; worker i computes i, i+P, i+2P, ...
 *                             (section "why a fixed task sequence tails").
 *   GEMM_SCHED_DYNAMIC        grid = all tiles (launch slots; see dynamic_grid for
 *                             the resident-only grid); every workgroup takes tiles
 *                             from atomic claim counters, the claim of the next tile
 *                             is prefetched through a ring of response records in
 *                             LDS (depth 3), a failed claim ends the worker, and
 *                             late-launched slots exit at once. This replaces the
 *                             hardware launch-cancel of the blog post (sections
 *                             "cancelling the launch ..." and "following the CUTLASS
 *                             source"), which gfx950 lacks.
 *
 * Claim counters of the dynamic mode (plan field claim_policy):
 *   0  one device-wide counter hands out every tile id in order: the pages' single
 *      work queue.
 *   1  (the default) eight counters, one per XCD: tile ids with id mod 8 == x form
 *      region x, the set a plain launch sends to XCD x. A worker claims from its
 *      own XCD's region and steals from the others once that is exhausted. Each
 *      counter returns each id of its region once, so exactly-once holds as with
 *      one counter; the worker's own-region tiles keep their operands in its
 *      XCD's L2 (MI355X has eight L2s; the pages' part has one).
 *   2  the same with contiguous regions (region x = the x-th of eight consecutive
 *      runs of ids), for grouped runs of small problems.
 *
 * Tail splitting (optional, tail_split >= 2; single GEMMs only). Whole tiles
 * quantise the finish: T = P + 1 tiles on P workers take two tile times. The
 * blog post names splitting work along K as what removes this and leaves it out
 * of its design (first section); here it is the work-unit decomposition of a
 * run: the tiles that fill whole waves of workers stay whole units, and each
 * of the r = T mod P tiles of the partial last wave (all T tiles when T < P)
 * becomes S units, K-chunks of nearly equal k-step counts. Every unit still has exactly one owner under
 * every scheduler. A chunk writes its fp32 partial tile to plan scratch; the
 * workgroup that completes a tile's last chunk adds the S partials in chunk
 * order (a fixed order: results do not depend on which chunk finished last)
 * and writes C. Split tiles therefore round differently from whole tiles.
 *
 * Layouts. Row-major and contiguous: A is M x K (lda = K), B is K x N (ldb = N),
 * C is M x N (ldc = N). bf16 is passed as raw 16-bit patterns. Device pointers
 * only (hipMalloc / torch device memory). A, B and C must be 16-byte aligned;
 * K and N must be multiples of 8 (16-byte rows); M is arbitrary. Edge tiles
 * (M, N, K not multiples of the tile) are handled by masking.
 *
 * Ownership. The caller owns A, B, C and keeps them alive until the stream has
 * passed the kernel. The plan (gemm_tile_cfg) owns all library scratch: the
 * claim counters, the tile log, the visit counters, the device status word,
 * the split tail's partial sums and the grouped-problem table. Runs are asynchronous and stream-ordered; nothing
 * here synchronises except gemm_sync, gemm_read_log, gemm_destroy and
 * gemm_test_spoiler's optional residency wait. Runs of one plan on different
 * streams are ordered on the device (a run waits for the plan's previous
 * stream). The plan keeps the stream of its last run: that stream must stay
 * valid until the plan's next run, gemm_sync, gemm_read_log or gemm_destroy,
 * which use it. A plan is not thread-safe.
 *
 * Graph capture. gemm_run and gemm_run_noalloc enqueue one kernel and nothing
 * else. A gemm_run made while its stream is capturing (hipStreamIsCapturing)
 * runs on a scheduler-state set of its own and leaves that state (claim
 * counters, gate, split-tile arrival counts) back at zero when it ends, so the
 * captured launch can be replayed any number of times; an uncaptured run skips
 * that clean-up, since the plan's next run clears the set it used (the clean-up
 * costs 2-4 us at the end of a launch). gemm_run_noalloc always cleans up after
 * itself. Make a plan's first run on the capture stream before capturing (a run
 * on a new stream first waits for the plan's previous stream with an event),
 * and gemm_run_noalloc's first call on a device outside capture (it clears its
 * state array then). With the tile log on, the visit counts of a captured
 * launch add up over its replays. A grouped run captures like a single one when
 * its problem table is the one the plan uploaded last (then it enqueues no
 * upload).
 *
 * Errors. Every call returns a gemm_status; 0 is success. Invalid arguments are
 * rejected before anything is enqueued. HIP failures return GEMM_E_HIP and the
 * HIP error text is kept in the plan (gemm_last_hip_error). Failures inside a
 * kernel (a gate wait that ran out, a ring protocol violation) are kept in the
 * plan's device status until gemm_sync or gemm_read_log returns them. Nothing
 * aborts and nothing throws across this boundary.
 */
#ifndef PTG_GEMM_H
#define PTG_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_status {
  GEMM_OK = 0,
  GEMM_E_INVALID_ARG = -1, /* null pointer, bad enum, bad descriptor field */
  GEMM_E_SHAPE = -2,       /* negative size, K or N not a multiple of 8, over a size limit */
  GEMM_E_UNSUPPORTED = -3, /* device is not gfx950, or an unsupported tile shape */
  GEMM_E_DEVICE = -4,      /* plan used while another device is current */
  GEMM_E_HIP = -5,         /* a HIP runtime call failed (see gemm_last_hip_error) */
  GEMM_E_NOMEM = -6,       /* device or pinned allocation failed */
  GEMM_E_TIMEOUT = -7,     /* a bounded wait ran out (spoiler residency, concurrency gate) */
  GEMM_E_SCHED = -8        /* the kernel flagged a claim-ring protocol violation */
} gemm_status;

typedef enum gemm_sched_mode {
  GEMM_SCHED_NONPERSISTENT = 0,
  GEMM_SCHED_STATIC = 1,
  GEMM_SCHED_DYNAMIC = 2
} gemm_sched_mode;

/* K orders (gemm_tile_desc.k_rotation). */
#define GEMM_KROT_AUTO 0
#define GEMM_KROT_OFF 1
#define GEMM_KROT_XCD 2
#define GEMM_KROT_XCD2 3
#define GEMM_KROT_UNIT 4

/* Launch grid of the dynamic mode (gemm_tile_desc.dynamic_grid). */
#define GEMM_GRID_ALL 0
#define GEMM_GRID_RESIDENT 1

/* Size limits (checked; GEMM_E_SHAPE beyond them). */
#define GEMM_MAX_K (1 << 20)
#define GEMM_MAX_N (1 << 22)
#define GEMM_MAX_M (1 << 30)
#define GEMM_MAX_TILES (1 << 30)
#define GEMM_MAX_TAIL_SPLIT 64
#define GEMM_TAIL_SPLIT_AUTO (-1) /* tail_split: the library picks the chunk count per run */
#define GEMM_MAX_CLAIM_GROUP 16

/*
 * Plan descriptor (a value type; gemm_create copies it). Fields:
 *   bm, bn, bk      output tile and K step: {128,128,32} or {256,256,32}
 *                   (the kernel stages 32-deep slices of K in a ring of four).
 *   ring_depth      depth of the LDS ring of claim records: 3 (2..3 accepted).
 *   claims_ahead    throttle: how many claims a dynamic worker holds beyond its
 *                   current tile: 0 (claim after finishing the tile), 1 or 2;
 *                   must be < ring_depth.
 *   claim_lead      with claims_ahead >= 1, the claims for later tiles are issued
 *                   at the start of k-step c = max(0, nk - claim_lead) of the
 *                   current tile (nk = its number of 32-deep k-steps); with
 *                   256 x 256 tiles at the start of the group of four k-steps
 *                   (counted from the tile's first) that holds c, i.e. one of
 *                   k-steps c - 3 .. c (the main loop runs four k-steps per trip
 *                   and claims only between trips). Late, so a worker does not
 *                   take work a not-yet-started slot would get, yet early enough
 *                   for the atomic's round trip to hide under the MFMAs. 0 = at
 *                   the last k-step (or group); >= nk = at the tile start.
 *   claim_policy    0 = one device-wide counter hands out tile ids in order.
 *                   1 = XCD-partitioned: tile ids with id mod 8 == x form region
 *                   x, handed out by counter x; a worker claims from the region
 *                   of the XCD it runs on and, when that is exhausted, steals
 *                   from the other regions. Every tile still has one owner; a
 *                   worker's own-region tiles keep their L2 locality.
 *                   2 = XCD-partitioned with contiguous regions: region x is
 *                   the x-th of eight consecutive runs of work-unit ids (in
 *                   claim order; the first U mod 8 runs one id longer), with
 *                   the same own-region-first claiming and stealing. Meant for
 *                   grouped runs of small problems, where it keeps each
 *                   problem's tiles, and so its A and B panels, on one XCD.
 *                   The failure-forcing preset (gemm_test_preset_counter)
 *                   applies to policy 0 only.
 *   raster          0 = row-major tile order; 1 = grouped-M with group height
 *                   raster_group tile rows.
 *   static_workers  static mode's P; 0 = resident workgroups (occupancy x CUs).
 *   log_capacity    work units to log per run; 0 turns the log off.
 *   min_lds_bytes   dynamic LDS padding per workgroup (limits residency; 0 = none).
 *   max_concurrent  0 = no cap; n > 0 lets at most n workgroups compute at once:
 *                   the "only 3 workers can run at the same time" condition of
 *                   the worked example in the blog post's section "why a fixed
 *                   task sequence tails". Reading taken: a device-side gate (an
 *                   atomic count of workgroups holding a slot), not a stream whose
 *                   CU mask leaves 3 compute units: this part sends workgroup w to
 *                   XCD w mod 8, and a mask that leaves whole XCDs without a CU
 *                   risks stalling the workgroups sent there. With min_lds_bytes
 *                   over half the CU's LDS each gated worker also owns its CU.
 *                   A workgroup waiting at the gate gives up after gate_spin_limit
 *                   polls; it then computes nothing and sets the plan's device
 *                   status to GEMM_E_TIMEOUT (gemm_sync, gemm_read_log). In the
 *                   static and non-persistent modes its tiles are then missing
 *                   from C; in the dynamic mode the other workers claim them.
 *   max_groups      capacity of the grouped-problem table (0 = 1024).
 *   device          HIP device ordinal; must be gfx950.
 *   tail_split      0 = off. GEMM_TAIL_SPLIT_AUTO (-1): split as below with a
 *                   chunk count the library picks per run: the largest power
 *                   of two up to 8 that gives every chunk an idle CU and at
 *                   least 64 k-steps (16 when fewer than 32 tiles split; four
 *                   times that for 128 x 128 tiles), 1 (no split) if none.
 *                   s in 2..GEMM_MAX_TAIL_SPLIT: split each tile of a
 *                   partial last wave into at most s K-chunks (fewer when the
 *                   idle workers or K, at >= 8 k-steps of bk a chunk, allow
 *                   fewer). Workers per wave: the static mode's P, else
 *                   occupancy x CUs. A run with fewer tiles than that is one
 *                   partial wave, so all its tiles split (on MI355X, 2048 x
 *                   2048 x 8192 with 256 x 256 tiles: 64 tiles, 4 chunks each,
 *                   140 -> 98 us). Off by default: with few k-steps a chunk
 *                   (K of 2048 or less) or with 128 x 128 tiles and as many
 *                   tiles as CUs, the partial sums cost more than they save.
 *                   gemm_create then reserves the partial-sum scratch:
 *                   bm x bn x 4 bytes per worker of one wave.
 *   group_order     grouped runs only: the order work units are handed out in.
 *                   0 = problem after problem, as given. 1 = problems with the
 *                   longest K first (stable for equal K): a tile's cost grows
 *                   with its K, and handing out the costly tiles first leaves
 *                   the cheap ones to fill the end of the run (the longest-
 *                   processing-time rule). With claim_policy 2 the sorted
 *                   problems are dealt to the eight regions in snake order
 *                   (regions 0..7, then 7..0, ...), the regions' lists placed
 *                   one after another, so every region starts with its share
 *                   of the longest problems. Tile ids in the log keep the
 *                   as-given numbering either way; unit ids follow the order.
 *   claim_group     single GEMMs only: tiles per work unit (0 or 1 = one tile;
 *                   up to GEMM_MAX_CLAIM_GROUP). One claim (one static step,
 *                   one non-persistent block) then takes g consecutive tile ids
 *                   of the raster order, run back to back by one worker: with
 *                   the grouped-M raster of height h and g = 2h the unit is a
 *                   2 x h block of tiles sharing A and B panels, the claim-sized
 *                   counterpart of a cluster. Exclusive with tail_split (a
 *                   claim group wins).
 *   b_layout        0 = B is K x N row-major (C = A . B, torch.matmul(A, B)).
 *                   1 = B is given as N x K row-major, i.e. the product is
 *                   C = A . B^T (torch.matmul(A, Bt.T)); its rows are K long,
 *                   so the same K % 8 and N % 8 rules apply. Applies to the
 *                   plan's single and grouped runs alike.
 *   gate_spin_limit polls of the concurrency gate before a waiting workgroup
 *                   gives up (0 = the default, about 4 million: a few seconds).
 *   k_rotation      the order a work unit walks its K range in (the sum is the
 *                   same; only the fp32 rounding order inside a tile changes,
 *                   and it depends on the unit id alone, so all schedulers give
 *                   bitwise the same C). When every workgroup walks K from the
 *                   same end, the concurrent reads of all CUs share their low
 *                   address bits (the same column of every row of A), which
 *                   holds memory bandwidth well below what the part streams
 *                   otherwise; a rotation (unit u starts part-way into its range
 *                   and wraps around) spreads them.
 *                   The phase follows a key: the unit id u in a single GEMM,
 *                   the problem's index in a grouped run (its tiles share its
 *                   operand panels and walk K together).
 *                   GEMM_KROT_AUTO (0, the default): per launch; for a single
 *                   GEMM two phases per XCD region with at most 8 tile columns
 *                   (each XCD then reads 32 distinct A panels at once), one
 *                   phase per region otherwise (an XCD's tiles share A panels,
 *                   which stay in step); for a grouped run a phase per problem.
 *                   GEMM_KROT_OFF: first k-step to last.
 *                   GEMM_KROT_XCD: key u starts at (u mod 8) / 8 of its range:
 *                   the eight XCD regions walk K at eight phases while the
 *                   workgroups of one XCD, which share operand panels through
 *                   its L2, stay together.
 *                   GEMM_KROT_XCD2: (u mod 16) / 16: two phases per region.
 *                   GEMM_KROT_UNIT: a phase per key (a hash of it).
 *                   Units whose K is not a multiple of 32 keep the plain order.
 *   dynamic_grid    the dynamic mode's grid. GEMM_GRID_ALL (0, the default):
 *                   one launch slot per work unit, as the blog post's
 *                   launch-cancel scheduler has; slots that start after every
 *                   unit is handed out exit at once. GEMM_GRID_RESIDENT: only as
 *                   many workgroups as can be resident at once (occupancy x CUs,
 *                   at most one per unit). Without launch cancel, the slots of
 *                   the full grid beyond the resident ones can only start as the
 *                   workers exit, and then leave again: about 1-3 us per launch
 *                   of 1024 tiles with the per-XCD counters (each late slot
 *                   probes every region before it leaves). The schedule
 *                   is the same either way (the counters decide who takes which
 *                   unit).
 */
typedef struct gemm_tile_desc {
  int32_t bm, bn, bk;
  int32_t ring_depth;
  int32_t claims_ahead;
  int32_t claim_lead;
  int32_t claim_policy;
  int32_t raster;
  int32_t raster_group;
  int32_t static_workers;
  int32_t log_capacity;
  int32_t min_lds_bytes;
  int32_t max_concurrent;
  int32_t max_groups;
  int32_t device;
  int32_t tail_split;
  int32_t group_order;
  int32_t claim_group;
  int32_t b_layout;
  int32_t gate_spin_limit;
  int32_t k_rotation;
  int32_t dynamic_grid;
} gemm_tile_desc;

/* Opaque plan: the tile_cfg argument of gemm_run. Owns all library scratch. */
typedef struct gemm_plan *gemm_tile_cfg;

/*
 * One log record (host copy) per work item, indexed by item id. An item is a
 * whole tile or one K-chunk of a split tile; without tail splitting the item
 * id is the tile id (in claim order for grouped runs with group_order = 1).
 * unit: the work unit (claim, static step, non-persistent block) that covered
 * the item, equal to the item id unless claim groups are on; tile: output
 * tile id in raster order (grouped: ids of problem g follow those of problems
 * < g); k_begin/k_end: the K range [k_begin, k_end) the item accumulated (the
 * whole K for a whole tile); worker: launch slot (blockIdx.x) that ran it;
 * hw_id / xcc_id: raw HW_ID and XCC_ID hardware registers of the wave that ran
 * it; t0/t1: s_memtime at item start / after its stores were issued; r0/r1:
 * the same moments on the constant-rate s_memrealtime clock (rate:
 * gemm_plan_info's wallclock_khz); visits: how many times the item was
 * finished (exactly-once => 1); problem: grouped problem index (0 otherwise).
 */
typedef struct gemm_tile_rec {
  uint32_t tile, worker, hw_id, xcc_id;
  uint64_t t0, t1, r0, r1;
  uint32_t visits, problem;
  uint32_t unit, k_begin, k_end, pad;
} gemm_tile_rec;

/* Facts about a plan and its last run. */
typedef struct gemm_plan_info {
  int32_t device;
  int32_t cu_count;          /* compute units */
  int32_t occupancy;         /* resident workgroups per CU for this plan's kernel */
  int32_t static_workers;    /* P the static mode uses for a large problem */
  int64_t wallclock_khz;     /* s_memrealtime rate */
  int64_t last_tiles;        /* T of the last run */
  int64_t last_units;        /* work units handed out in the last run */
  int64_t last_items;        /* work items (log records) of the last run: tiles plus split chunks */
  int64_t last_split_base;   /* first split tile (== last_tiles when nothing was split) */
  int32_t last_split_chunks; /* K-chunks per split tile (1 when nothing was split) */
  int32_t last_claim_group;  /* tiles per unit of the last run */
  int64_t last_grid;         /* grid size of the last run */
  int32_t last_mode;         /* scheduler of the last run (-1 before the first) */
  int32_t lds_bytes;         /* LDS per workgroup */
  int32_t last_k_rotation;   /* K order of the last run as resolved: GEMM_KROT_OFF, _XCD, _XCD2 or _UNIT */
  int32_t pad;
} gemm_plan_info;

/*
 * Fill *out with the defaults for a square tile edge of 128 or 256 on `device`:
 * ring depth 3 and one claim ahead (the response pipeline depth and throttle of
 * the blog post's section "following the CUTLASS source"), per-XCD claim
 * counters, log off. Errors: GEMM_E_INVALID_ARG (out NULL), GEMM_E_UNSUPPORTED
 * (another edge). No HIP call.
 */
gemm_status gemm_default_desc(gemm_tile_desc *out, int32_t tile_edge, int32_t device);

/*
 * Validate *desc and build a plan on desc->device, which must be the current
 * device. The plan is the scheduler configuration of the task-scheduling guide
 * ("CUTLASS Task Scheduling resources", section "TileSchedulerConfig": the
 * scheduler type and its parameters are fixed before launch) together with all
 * device scratch a run needs: the claim counters, the tile log and visit
 * counters, the grouped-problem table and, with tail_split, the partial-sum
 * workspace. All allocation happens here, none in gemm_run. *out receives the
 * plan (NULL on failure). Errors: GEMM_E_INVALID_ARG (a field out of range, or
 * LDS padding beyond the device limit), GEMM_E_UNSUPPORTED (not gfx950 - the
 * capability check of "B200 Cluster Persistent Scheduler", section "B -
 * boundaries" - or an unsupported tile), GEMM_E_DEVICE (desc->device is not
 * current), GEMM_E_NOMEM, GEMM_E_HIP.
 */
gemm_status gemm_create(gemm_tile_cfg *out, const gemm_tile_desc *desc);

/*
 * Enqueue C = A.B on `stream` (a hipStream_t; NULL = the null stream) with
 * scheduler `sched_mode`, one of the three modes of the blog post's table in
 * the section "from one tile per block to one worker computing continuously"
 * (see the top of this file). A: M x K bf16, B: K x N bf16, C: M x N fp32, all
 * device pointers. M == 0 or N == 0 enqueues nothing; K == 0 writes zeros.
 * Exactly one kernel launch; no allocation, no host synchronisation. If the
 * plan's previous run was enqueued on another stream, the run first waits on
 * the device for that stream's work (the plan's scratch serves one run at a
 * time). Errors (returned before anything is enqueued): GEMM_E_INVALID_ARG (a
 * NULL pointer for a non-empty problem, pointers not 16-byte aligned, a bad
 * mode), GEMM_E_SHAPE (negative sizes, K or N not a multiple of 8, over a size
 * limit), GEMM_E_DEVICE (another device is current); GEMM_E_HIP if the launch
 * fails. Failures inside the kernel are reported later by gemm_sync or
 * gemm_read_log.
 */
gemm_status gemm_run(const void *A, const void *B, float *C, int64_t M, int64_t N, int64_t K,
                     int32_t sched_mode, gemm_tile_cfg tile_cfg, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The same product as
 * gemm_run with the plan gemm_default_desc(256) gives (256 x 256 tiles,
 * per-XCD claim counters, one claim ahead, automatic K order, log off, no
 * split tail, no claim groups, no concurrency gate, B as K x N), with no plan: the scheduler state
 * lives in a library-owned device array of 8960 bytes per device (two control
 * sets and a status word), which each device keeps until the process ends. Its
 * size does not depend on M, N or K; sizes beyond the library limits are
 * refused (GEMM_E_SHAPE) as by gemm_run. The first call on a device enqueues,
 * before the GEMM, a small kernel that clears the array. Calls never allocate,
 * free or synchronise.
 * All calls on one device share that array, and each call leaves the next
 * call's control set cleared: calls on one device must not overlap (enqueue
 * them on one stream, or order them); overlapping calls race on the claim
 * counters. d_status (optional, 4-byte aligned device pointer, caller-owned
 * and caller-cleared) receives the error bits a plan's gemm_sync would report
 * (bit 1: a claim-ring record for the wrong ordinal; the gate bit cannot occur
 * without a gate); with NULL they go to the array's own status word, which no
 * call reports. Errors: as gemm_run, plus GEMM_E_UNSUPPORTED (current device
 * not gfx950) and GEMM_E_INVALID_ARG (misaligned d_status).
 */
gemm_status gemm_run_noalloc(const void *A, const void *B, float *C, int64_t M, int64_t N, int64_t K,
                             int32_t sched_mode, uint32_t *d_status, void *stream);

/*
 * Grouped variant: G independent problems C_g = A_g.B_g in one launch, their
 * tiles numbered problem after problem: the uneven-cost work the "B200 Cluster
 * Persistent Scheduler" page sends to the dynamic scheduler (section "E -
 * executable steps", choosing the scheduling mode). A, B, C, M, N, K are host
 * arrays of length G (copied before return; the caller may free them). Each
 * problem follows the single-GEMM rules. G <= the plan's max_groups, else
 * GEMM_E_SHAPE; G <= 0 or a NULL array is GEMM_E_INVALID_ARG. The problem
 * table is copied to the device on `stream` (from the plan's pinned staging)
 * only when it differs from the last one.
 */
gemm_status gemm_run_grouped(int32_t G, const void *const *A, const void *const *B, float *const *C,
                             const int64_t *M, const int64_t *N, const int64_t *K,
                             int32_t sched_mode, gemm_tile_cfg tile_cfg, void *stream);

/*
 * Synchronise the last run's stream and copy its log to host_out (up to cap
 * records, in unit-id order, including units that never ran: visits == 0; for
 * those, tile and k_begin/k_end are what the launch planned and worker is
 * 0xFFFFFFFF). The log is the per-tile ownership record whose exactly-once
 * property the blog post's section "cancelling the launch, receiving the work
 * coordinate" states (each tile owned by one worker). *n_out receives the
 * number of records written (0 with the log off). Returns the device status as
 * gemm_sync does, also when the log is off; the log is still copied.
 */
gemm_status gemm_read_log(gemm_tile_cfg tile_cfg, gemm_tile_rec *host_out, size_t cap, size_t *n_out);

/*
 * Synchronise the plan's last stream and return the device-side status of every
 * run since the previous gemm_sync or gemm_read_log, then clear it. A failure
 * must be observable ("CUTLASS Cluster Launch Control dynamic persistent kernel",
 * section "cluster granularity and exit after failure"): GEMM_E_TIMEOUT if a
 * workgroup gave up waiting at the concurrency gate (it computed nothing; in
 * the static and non-persistent modes its tiles are missing from C),
 * GEMM_E_SCHED if a consumer found a claim-ring record for the wrong ordinal.
 * GEMM_OK before the first run. GEMM_E_HIP if the synchronisation fails.
 */
gemm_status gemm_sync(gemm_tile_cfg tile_cfg);

/* Read plan facts. */
gemm_status gemm_plan_info_get(gemm_tile_cfg tile_cfg, gemm_plan_info *out);

/*
 * Release the plan and its scratch (synchronises its last stream first). NULL is
 * a no-op. Device status not yet read is discarded.
 */
gemm_status gemm_destroy(gemm_tile_cfg tile_cfg);

/* Static text for a status code. */
const char *gemm_status_str(int32_t status);

/* Text of the last HIP error seen by this plan ("" if none). */
const char *gemm_last_hip_error(gemm_tile_cfg tile_cfg);

/*
 * Failure forcing for tests: the next dynamic run starts its claim counter at
 * `start` instead of 0, so exactly tiles start..T-1 are computed and every
 * worker's claims fail once the counter passes T-1 (a claim fails when no work
 * is left: blog post, section "cluster granularity and exit after failure").
 */
gemm_status gemm_test_preset_counter(gemm_tile_cfg tile_cfg, uint32_t start);

/*
 * Failure forcing for tests: the next run of a plan with max_concurrent > 0
 * starts with `held` of its gate slots counted as taken. With held >=
 * max_concurrent every workgroup's bounded wait runs out (after the plan's
 * gate_spin_limit polls), every workgroup exits without computing, and
 * gemm_sync reports GEMM_E_TIMEOUT: the failure path of the blog post's section
 * "cluster granularity and exit after failure", forced from the host so the
 * kernel still ends normally.
 */
gemm_status gemm_test_preset_gate(gemm_tile_cfg tile_cfg, uint32_t held);

/*
 * Test helper: create a stream on `device` (current) whose kernels may only use
 * the compute units set in `mask` (words x 32 bits, hipExtStreamCreateWithCUMask)
 * and return it in *out_stream; release it with gemm_test_stream_destroy. This is
 * the other reading of the worked example's concurrency cap (a CU mask; the plan's
 * gate is the one the library uses, see max_concurrent): a mask must leave compute
 * units on every XCD, since workgroups are sent to XCDs in turn. Errors:
 * GEMM_E_INVALID_ARG (NULL, no unit named, a unit beyond the device's, more
 * than 64 words), GEMM_E_DEVICE, GEMM_E_UNSUPPORTED (not gfx950), GEMM_E_HIP.
 */
gemm_status gemm_test_stream_cu_mask(void **out_stream, int32_t device, const uint32_t *mask, uint32_t words);

/* Destroy a stream made by gemm_test_stream_cu_mask. */
gemm_status gemm_test_stream_destroy(void *stream);

/*
 * Occupy `n_wgs` compute units for `spin_ns` nanoseconds on `stream`: each
 * workgroup takes a whole CU's LDS, records {s_memrealtime at start, HW_ID,
 * XCC_ID, end} into d_log (4 uint64 per workgroup; may be NULL) and spins on the
 * constant-rate clock until its time is up (a bounded wait). This is the
 * "some SMs are occupied by another kernel" scenario of the blog post's section
 * "why a fixed task sequence tails". If wait_resident_ms > 0 the call returns
 * only once all n_wgs workgroups have started, or GEMM_E_TIMEOUT after that
 * many milliseconds (the spoiler still ends on its own).
 */
gemm_status gemm_test_spoiler(int32_t device, int32_t n_wgs, int64_t spin_ns, void *stream,
                              uint64_t *d_log, double wait_resident_ms);

/*
 * Measurement helper (no page behind it; a fact about the part): run an
 * MFMA-only kernel on `device`, one workgroup of four waves per CU, each wave
 * issuing `iters` rounds of independent bf16 MFMAs with no memory traffic:
 * eight v_mfma_f32_32x32x16_bf16 (mfma_block == 32, the 128 x 128 tiles'
 * instruction) or sixteen v_mfma_f32_16x16x32_bf16 (mfma_block == 16, the
 * 256 x 256 tiles' instruction) per round, the same flops either way; operands
 * constant (random_operands == 0) or differing from one MFMA to the next
 * (pseudo-random bf16). Synchronous: it allocates a small scratch buffer, times
 * the launch with events and frees the buffer. Outputs: *tflops_out, the dense
 * bf16 rate achieved, and *clock_ghz_out, the mean shader clock during the run
 * (s_memtime over s_memrealtime ticks). iters must be in 1..10^7 and
 * mfma_block 16 or 32, else GEMM_E_INVALID_ARG.
 */
gemm_status gemm_mfma_probe(int32_t device, int32_t iters, int32_t random_operands, int32_t mfma_block,
                            double *tflops_out, double *clock_ghz_out);

/*
 * Measurement helper (no page behind it; a fact about the part): the memory
 * bandwidth a plain streaming kernel reaches on `device` (current), the
 * practical ceiling beside the 8 TB/s data-sheet figure for the HBM-bound GEMM
 * shapes. kind 0: read `bytes` once (16-byte non-temporal loads per lane,
 * grid-stride, four workgroups of 256 threads per CU); kind 1: copy `bytes`
 * (read and write, the same access). Synchronous: allocates its buffers (one,
 * or two for a copy, of `bytes` each; the buffer is zero-filled), runs 3
 * untimed and `reps` timed launches between events and frees them.
 * *gbs_out receives bytes moved (read, or read + written) per second in GB/s.
 * bytes must be a multiple of 4096 in [1 MiB, 16 GiB], reps in 1..1000, else
 * GEMM_E_INVALID_ARG; GEMM_E_NOMEM if the buffers do not fit.
 */
gemm_status gemm_hbm_probe(int32_t device, int64_t bytes, int32_t kind, int32_t reps, double *gbs_out);

#ifdef __cplusplus
}
#endif

#endif /* PTG_GEMM_H */

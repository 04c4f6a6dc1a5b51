"""CPU oracle for the persistent tiled GEMM and its tile schedulers.

TEST INFRASTRUCTURE ONLY. The product path never imports this package: only the
test suite, the smoke check and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library. Its only input source is ``workloads``,
which draws random numbers and holds none of the arithmetic computed here.

Modules
  gemm_ref    C = A.B on the exact bf16 inputs, accumulated in float64, and the
              acceptance test a GPU result must pass.
  sched_model discrete-event model of the three tile schedulers (non-persistent,
              static grid-stride, dynamic claim) over execution slots.
  ring_model  exhaustive interleaving checker for the claim / prefetch-ring protocol.
  ownership   checks of a per-tile ownership log (exactly once, per-mode owner rules).

Every function cites the passage of the source pages it follows. A page is named
by its title; the pages are:
  [CLC]  "CUTLASS Blackwell Cluster Launch Control dynamic persistent kernel" (blog post)
  [TS]   "CUTLASS Task Scheduling resources: PipelineConfig, MemoryResource and WorkQueue"
  [SKILL] "B200 Cluster Persistent Scheduler" (agent-skill listing)
"""

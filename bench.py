#!/usr/bin/env python3
"""Benchmark: bf16 GEMM TFLOP/s and % of MFMA peak on 8192^3; tail makespans.

One step = one pass of the whole hot path: a gemm_run of the dynamic scheduler
(atomic claim counters + LDS claim ring) on M = N = K = 8192, 256x256 tiles (K staged 32 deep,
automatic K order), A and B i.i.d. N(0,1)/sqrt(K) in bf16, fp32 C, tile log on. Inputs are
resident in HBM before timing starts. The kernel time is measured with HIP events on
the stream the kernel is launched on.

Printed: ONE JSON line with the contract fields, a `roofline` object for the
GEMM kernel, a `cpu_baseline` object (the CPU oracle timed on a bounded row
sample of the same workload), the static / non-persistent modes at the same
shape, and (unless --no-tail) the tail makespans of the partial-occupancy,
uneven-cost grouped, tail-boundary and worked-example workloads.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "bf16 GEMM TFLOP/s and % MFMA peak; tail makespan static vs dynamic"
KERNEL_SOURCES = ("persistent_tiled_gemm_amd/csrc/gemm_kernel.hip", "persistent_tiled_gemm_amd/csrc/ptg_device.hpp",
                  "persistent_tiled_gemm_amd/csrc/ptg_internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_square_8192_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(launch_units: float):
    """HBM bytes per launch from the committed counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def time_runs(fn, steps: int, warmup: int, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def time_interleaved(fns, rounds: int, per_round: int, stream, warm: int = 10):
    """Mean ms per call of each function, timed in `rounds` blocks of `per_round` calls per function,
    the order of the functions alternating between rounds; each block starts with three untimed calls
    (the first call after a switch or an idle gap reads slow). Before the first block every function
    runs `warm` times: the first launches over freshly allocated operands read several percent slow
    (measured on the tail-boundary shape: 153-165 us against 144-148 us from then on)."""
    import torch
    total = {k: 0.0 for k in fns}
    names = list(fns)
    for k in names:
        for _ in range(warm):
            fns[k]()
    torch.cuda.synchronize()
    for r in range(rounds):
        for k in (names if r % 2 == 0 else names[::-1]):
            total[k] += time_runs(fns[k], per_round, 3, stream) * per_round
    return {k: total[k] / (rounds * per_round) for k in names}


def cu_key(hw_id, xcc_id):
    """Physical CU identity from the HW_ID register (cu, sh, se fields, bits 8..15) and the XCC id."""
    return (xcc_id.astype(np.int64) << 8) | ((hw_id.astype(np.int64) >> 8) & 0xFF)


def makespan_from_log(rec, khz):
    ran = rec[rec["visits"] > 0]
    if len(ran) == 0:
        return None
    r0 = ran["r0"].astype(np.float64)
    r1 = ran["r1"].astype(np.float64)
    span_us = (r1.max() - r0.min()) / khz * 1e3
    dur_us = (r1 - r0) / khz * 1e3
    return {"makespan_us": span_us, "tile_median_us": float(np.median(dur_us)), "tiles": int(len(ran)),
            "workers": int(len(np.unique(ran["worker"]))), "cus": int(len(np.unique(cu_key(ran["hw_id"], ran["xcc_id"]))))}


def clock_from_log(rec, khz):
    """Mean shader clock (GHz) over the logged items of a run: s_memtime cycles over s_memrealtime ticks."""
    ran = rec[rec["visits"] > 0]
    if len(ran) == 0:
        return None
    cyc = (ran["t1"] - ran["t0"]).astype(np.float64)
    wall = (ran["r1"] - ran["r0"]).astype(np.float64)
    ok = wall > 0
    return float(np.sum(cyc[ok]) / np.sum(wall[ok]) * khz * 1e-6)


def median_run(run_and_read, khz, n: int = 3):
    """Call run_and_read() n times (it runs one launch, waits for it and returns (log records, extra
    fields)); return the makespan summary of the run with the median makespan, with every run's
    makespan listed."""
    runs = []
    for _ in range(n):
        rec, extra = run_and_read()
        ms = makespan_from_log(rec, khz)
        ms.update(extra)
        runs.append((ms["makespan_us"], ms, rec))
    runs.sort(key=lambda x: x[0])
    _, ms, rec = runs[len(runs) // 2]
    ms["makespan_us_runs"] = [round(x[0], 2) for x in runs]
    return ms, rec


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def blas_info():
    """(threads, vendor string) of the BLAS numpy calls: threadpoolctl's view of the loaded library,
    else numpy's build configuration."""
    threads, vendor = None, None
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            threads = max(int(i.get("num_threads", 1)) for i in blas)
            vendor = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')} "
                               f"threading, {i.get('architecture', '?')})" for i in blas)
    except Exception:  # pragma: no cover
        pass
    if vendor is None:
        try:
            cfg = np.show_config(mode="dicts")
            b = cfg["Build Dependencies"]["blas"]
            vendor = f"{b.get('name')} {b.get('version')}"
        except Exception:  # pragma: no cover
            vendor = "unknown"
    return threads, vendor


def cpu_baseline(problem, target_s: float = 10.0):
    """Time the CPU oracle (gemm_ref_rows: exact bf16 decode + fp64 product) on a row sample."""
    from oracle.gemm_ref import gemm_ref_rows
    threads, vendor = blas_info()
    affinity = len(os.sched_getaffinity(0))
    if threads is None:
        threads = affinity
    M, K = problem.a_bits.shape
    N = problem.b_bits.shape[1]
    rows = 256
    t0 = time.perf_counter()
    gemm_ref_rows(problem.a_bits, problem.b_bits, range(rows))
    t = time.perf_counter() - t0
    rows = int(min(M, max(256, rows * target_s / max(t, 1e-3))))
    t0 = time.perf_counter()
    gemm_ref_rows(problem.a_bits, problem.b_bits, range(rows))
    t = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} of {M} rows of C (all {N} columns, K={K}), fp64, {t:.2f} s",
            "cores_note": "BLAS threads the fp64 product ran on (the decode is single-threaded NumPy)",
            "affinity_cpus": affinity, "blas": vendor, "cpu_model": host_cpu_model(),
            "fp64_gflops": flops / t / 1e9, "wall_s": t}


def run_tail_sections(ptg, torch, stream, khz, square):
    """Makespans per scheduler on the partial-occupancy, grouped, tail-boundary and worked-example workloads."""
    from workloads import make_workload
    out = {}
    modes = ("nonpersistent", "static", "dynamic")

    # partial occupancy: 8192^3 co-run with a 64-CU spoiler spinning 2 ms
    log("tail: partial occupancy")
    p, A, B, C = square
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024)
    spoil_stream = torch.cuda.Stream()
    res = {}
    def co_run(mode):
        spoiler_log = torch.zeros(64 * 4, dtype=torch.int64, device="cuda")
        ptg.gemm_test_spoiler(64, 2_000_000, stream=spoil_stream, log=spoiler_log, wait_resident_ms=2000.0)
        ptg.gemm_run(A, B, C, plan, mode=mode, stream=stream)
        torch.cuda.synchronize()
        rec = ptg.gemm_read_log(plan)
        sl = spoiler_log.cpu().numpy().reshape(64, 4).astype(np.float64)
        ran = rec[rec["visits"] > 0]
        return rec, {"spoiler_cus": int(len(np.unique(cu_key(sl[:, 2].astype(np.int64), sl[:, 3].astype(np.int64))))),
                     "spoiler_end_after_first_tile_us": float((sl[:, 1].max() - ran["r0"].min()) / khz * 1e3)}
    for mode in modes:
        ptg.gemm_run(A, B, C, plan, mode=mode, stream=stream)  # warm
        torch.cuda.synchronize()
        res[mode], _ = median_run(lambda: co_run(mode), khz)
    # each mode in its own median tile time (under the spoiler the dynamic run's
    # tiles take longer than the static run's, a memory effect, not scheduling)
    for mode in modes:
        res[mode]["makespan_t"] = res[mode]["makespan_us"] / res[mode]["tile_median_us"]
    res["dynamic_beats_static"] = bool(res["dynamic"]["makespan_us"] < res["static"]["makespan_us"])
    out["partial_occupancy"] = res
    plan.destroy()

    # uneven-cost grouped: 64 x (1024 x 1024, K_g = 512 U{1..16})
    log("tail: grouped uneven")
    w = make_workload("grouped_uneven")
    As = [ptg.bf16_from_bits(q.a_bits) for q in w.problems]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in w.problems]
    Cs = [torch.empty((q.M, q.N), dtype=torch.float32, device="cuda") for q in w.problems]
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024)
    res = {}
    ks = np.array([q.K for q in w.problems])
    # the dynamic scheduler handing out the longest-K problems first, beside the three modes
    lplan = ptg.gemm_create(tile_edge=256, log_capacity=1024, group_order=1)
    # the same order dealt to contiguous XCD regions (each XCD runs whole problems)
    cplan = ptg.gemm_create(tile_edge=256, log_capacity=1024, group_order=1, claim_policy=2)
    variants = {mode: (mode, plan) for mode in modes}
    variants["dynamic_longest_k_first"] = ("dynamic", lplan)
    variants["dynamic_longest_k_first_contiguous_regions"] = ("dynamic", cplan)
    fns = {name: (lambda mode=mode, pl=pl: ptg.gemm_run_grouped(As, Bs, Cs, pl, mode=mode, stream=stream))
           for name, (mode, pl) in variants.items()}
    kernel_ms = time_interleaved(fns, rounds=4, per_round=5, stream=stream)

    def logged(fn, pl):
        fn()
        torch.cuda.synchronize()
        return ptg.gemm_read_log(pl), {}
    for name, (mode, pl) in variants.items():
        ms, rec = median_run(lambda: logged(fns[name], pl), khz)
        ms["kernel_ms"] = kernel_ms[name]
        ms["tflops"] = w.flops / (kernel_ms[name] * 1e-3) / 1e12
        res[name] = ms
        if name == "static":
            ran = rec[rec["visits"] > 0]
            dur = ((ran["r1"] - ran["r0"]).astype(np.float64) / khz * 1e3)
            kt = ks[ran["problem"]] / 32.0   # 32-deep k-steps, the kernel's unit of K
            alpha, beta = np.polyfit(kt, dur, 1)
    res["cost_fit_us"] = {"per_kstep": float(alpha), "fixed": float(beta)}
    lplan.destroy()
    cplan.destroy()
    res["dynamic_beats_static"] = bool(res["dynamic"]["makespan_us"] < res["static"]["makespan_us"])
    out["grouped_uneven"] = res
    plan.destroy()
    del As, Bs, Cs

    # tail boundary: T = 255 / 256 / 257 tiles of 256 x 256, K = 4096
    log("tail: boundary")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=512)
    res = {}
    for name in ("tail_255", "tail_256", "tail_257"):
        q = make_workload(name).problems[0]
        A = ptg.bf16_from_bits(q.a_bits)
        B = ptg.bf16_from_bits(q.b_bits)
        C = torch.empty((q.M, q.N), dtype=torch.float32, device="cuda")
        variants = {mode: (mode, plan) for mode in modes}
        splan = aplan = None
        if name == "tail_257":
            # the one tile of the partial last wave split into (at most 4) K-chunks over idle workers,
            # and with the chunk count the library picks
            splan = ptg.gemm_create(tile_edge=256, log_capacity=512, tail_split=4)
            aplan = ptg.gemm_create(tile_edge=256, log_capacity=512, tail_split=ptg.TAIL_SPLIT_AUTO)
            variants["static_tail_split"] = ("static", splan)
            variants["dynamic_tail_split"] = ("dynamic", splan)
            variants["dynamic_tail_split_auto"] = ("dynamic", aplan)
        fns = {v: (lambda mode=mode, pl=pl: ptg.gemm_run(A, B, C, pl, mode=mode, stream=stream))
               for v, (mode, pl) in variants.items()}
        kernel_ms = time_interleaved(fns, rounds=4, per_round=5, stream=stream)

        def logged(fn, pl):
            fn()
            torch.cuda.synchronize()
            return ptg.gemm_read_log(pl), {}
        r = {}
        for v, (mode, pl) in variants.items():
            ms, _ = median_run(lambda: logged(fns[v], pl), khz)
            ms["kernel_us"] = kernel_ms[v] * 1e3
            if pl is plan:
                ms["hbm_gbs"] = (q.M * q.K * 2 + q.K * q.N * 2 + q.M * q.N * 4) / (kernel_ms[v] * 1e-3) / 1e9
            else:
                info = ptg.gemm_plan_info_get(pl)
                ms["units"] = int(info["last_units"])
                ms["chunks"] = int(info["last_split_chunks"])
                ms["makespan_t"] = ms["makespan_us"] / r[mode]["tile_median_us"]
            r[v] = ms
        if splan is not None:
            splan.destroy()
            aplan.destroy()
        res[name] = r
        del A, B, C
    out["tail_boundary"] = res
    plan.destroy()

    # worked example: 12 tiles of 128 x 128, at most 3 workers at once, static P = 4; one
    # work queue (the single claim counter), as in the example
    log("tail: worked example")
    q = make_workload("worked_example").problems[0]
    A = ptg.bf16_from_bits(q.a_bits)
    B = ptg.bf16_from_bits(q.b_bits)
    C = torch.empty((q.M, q.N), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=128, log_capacity=64, max_concurrent=3, static_workers=4, claim_policy=0,
                           min_lds_bytes=96 * 1024)
    res = {}

    def logged_we(mode):
        ptg.gemm_run(A, B, C, plan, mode=mode, stream=stream)
        torch.cuda.synchronize()
        return ptg.gemm_read_log(plan), {}
    we_logs = {}
    for mode in modes:
        for _ in range(2):
            ptg.gemm_run(A, B, C, plan, mode=mode, stream=stream)
        res[mode], we_logs[mode] = median_run(lambda: logged_we(mode), khz, n=5)
    # makespan in units of each mode's own median tile time (the pages' t)
    for mode in modes:
        res[mode]["makespan_t"] = res[mode]["makespan_us"] / res[mode]["tile_median_us"]
    res["static_over_dynamic"] = res["static"]["makespan_us"] / res["dynamic"]["makespan_us"]
    # the two overheads the pages' hand calculation leaves out, from the logs of the median runs:
    # the gate handoff (non-persistent: the (k+3)-th start follows the k-th end) and the exposed
    # per-tile claim cost (dynamic: gaps between a worker's consecutive tiles)
    np_rec, dyn_rec = we_logs["nonpersistent"], we_logs["dynamic"]
    r0 = np.sort(np_rec["r0"].astype(np.float64))
    r1 = np.sort(np_rec["r1"].astype(np.float64))
    handoff_us = float(np.median((r0[3:] - r1[:-3]) / khz * 1e3))
    gaps = []
    for w in np.unique(dyn_rec["worker"]):
        mine = dyn_rec[dyn_rec["worker"] == w]
        mine = mine[np.argsort(mine["r0"])]
        gaps += ((mine["r0"][1:].astype(np.float64) - mine["r1"][:-1].astype(np.float64)) / khz * 1e3).tolist()
    claim_gap_us = float(np.median(gaps)) if gaps else 0.0
    res["overheads_us"] = {"gate_handoff_l": handoff_us, "claim_gap_k": claim_gap_us}
    t_np, t_st, t_dy = (res[m]["tile_median_us"] for m in ("nonpersistent", "static", "dynamic"))
    res["with_overheads_t"] = {"nonpersistent": (4 * t_np + 3 * handoff_us) / t_np,
                               "static": (6 * t_st + handoff_us) / t_st,
                               "dynamic": (4 * t_dy + 3 * claim_gap_us) / t_dy}
    res["pages_hand_calc_t"] = {"static": 6, "dynamic": 4, "nonpersistent": 4}
    out["worked_example"] = res
    plan.destroy()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--mode", default="dynamic", choices=["nonpersistent", "static", "dynamic"])
    ap.add_argument("--claims-ahead", type=int, default=1)
    ap.add_argument("--claim-policy", type=int, default=1, choices=[0, 1, 2],
                    help="0: one device-wide claim counter; 1: per-XCD counters with stealing (interleaved "
                         "regions); 2: the same with contiguous regions (the 8192^3 line takes 0 or 1)")
    ap.add_argument("--group-order", type=int, default=0, choices=[0, 1],
                    help="grouped workloads under --profile-workload: 1 = longest K first")
    ap.add_argument("--raster-group", type=int, default=0, help="grouped-M raster height (0: row-major)")
    ap.add_argument("--no-log", action="store_true", help="turn the tile log off")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tail", action="store_true")
    ap.add_argument("--no-modes", action="store_true", help="skip timing the other schedulers")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times, for the byte counters' scale), then "
                         "time 20 more: the practical HBM ceiling")
    ap.add_argument("--trace-out", default="", metavar="PATH",
                    help="write the last timed headline launch's tile log as a Chrome trace (one event per tile "
                         "on the timeline of the CU that ran it)")
    ap.add_argument("--dispatch-clocks", action="store_true",
                    help="only run the headline launches (--warmup + --steps, back to back, each on a plan of its "
                         "own so every launch keeps its tile log) and print each launch's time and shader clock")
    ap.add_argument("--profile-workload", default="", metavar="NAME",
                    choices=["", "tail_255", "tail_256", "tail_257", "grouped_uneven"],
                    help="only run that workload (--steps times, after --warmup) for a profiler; "
                         "prints its timing and algorithmic HBM rate, not the benchmark line")
    args = ap.parse_args()
    if args.claim_policy == 2 and not args.profile_workload:
        ap.error("--claim-policy 2 applies to --profile-workload runs only")

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(only the single-GPU path is measured).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.profile_workload:
        import persistent_tiled_gemm_amd as ptg
        from workloads import make_workload
        ptg.load_library()
        probs = make_workload(args.profile_workload).problems
        As = [ptg.bf16_from_bits(q.a_bits) for q in probs]
        Bs = [ptg.bf16_from_bits(q.b_bits) for q in probs]
        Cs = [torch.empty((q.M, q.N), dtype=torch.float32, device="cuda") for q in probs]
        plan = ptg.gemm_create(tile_edge=256, claim_policy=args.claim_policy, group_order=args.group_order,
                               log_capacity=0 if args.no_log else 1024)
        stream = torch.cuda.current_stream()
        if len(probs) == 1:
            fn = lambda: ptg.gemm_run(As[0], Bs[0], Cs[0], plan, mode=args.mode, stream=stream)
        else:
            fn = lambda: ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=args.mode, stream=stream)
        ms = time_runs(fn, args.steps, args.warmup, stream)
        nbytes = sum(q.M * q.K * 2 + q.K * q.N * 2 + q.M * q.N * 4 for q in probs)
        flops = sum(2.0 * q.M * q.N * q.K for q in probs)
        print(json.dumps({"workload": args.profile_workload, "mode": args.mode, "claim_policy": args.claim_policy,
                          "group_order": args.group_order, "ms": ms,
                          "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / (ms * 1e-3) / 1e9,
                          "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "tflops": flops / (ms * 1e-3) / 1e12}), flush=True)
        plan.destroy()
        return
    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        # timing (a profiler run counts the first 5 launches only: it filters on nothing, so keep them first)
        stream = torch.cuda.current_stream()
        ms = time_runs(lambda: dst.copy_(src), 20, 0, stream)
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 25,
                          "copy_ms": ms, "copy_gbs_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)
        return
    import persistent_tiled_gemm_amd as ptg
    from workloads import make_workload

    ptg.load_library()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    log("generating square_8192 inputs")
    w = make_workload("square_8192")
    p = w.problems[0]
    M, N, K = p.M, p.N, p.K
    A = ptg.bf16_from_bits(p.a_bits)
    B = ptg.bf16_from_bits(p.b_bits)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fields = {"tile_edge": 256, "claims_ahead": args.claims_ahead, "claim_policy": args.claim_policy,
              "log_capacity": 0 if args.no_log else 1024}
    if args.raster_group > 1:
        fields.update(raster=1, raster_group=args.raster_group)
    plan = ptg.gemm_create(**fields)
    info = ptg.gemm_plan_info_get(plan)
    khz = info["wallclock_khz"]
    flops = 2.0 * M * N * K

    if args.dispatch_clocks:
        # the headline's launches, back to back as timed, each on its own plan (so each keeps its log):
        # per launch the kernel time (events around each launch) and the clock its tiles ran at
        n = args.warmup + args.steps
        plans = [ptg.gemm_create(**dict(fields, log_capacity=1024)) for _ in range(n)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i, pl in enumerate(plans):
            ptg.gemm_run(A, B, C, pl, mode=args.mode, stream=stream)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        for i, pl in enumerate(plans):
            rec = ptg.gemm_read_log(pl)
            ran = rec[rec["visits"] > 0]
            cyc = (ran["t1"] - ran["t0"]).astype(np.float64)
            print(json.dumps({"launch": i + 1, "timed": i >= args.warmup, "us": evs[i].elapsed_time(evs[i + 1]) * 1e3,
                              "clock_ghz": clock_from_log(rec, khz), "tile_cycles_median": float(np.median(cyc)),
                              "makespan_us": makespan_from_log(rec, khz)["makespan_us"]}), flush=True)
            pl.destroy()
        plan.destroy()
        return

    log(f"timing {args.mode}: warmup {args.warmup}, steps {args.steps}")
    ms = time_runs(lambda: ptg.gemm_run(A, B, C, plan, mode=args.mode, stream=stream), args.steps, args.warmup, stream)
    tflops = flops / (ms * 1e-3) / 1e12
    clock_ghz = None
    if not args.no_log:
        last_log = ptg.gemm_read_log(plan)
        clock_ghz = clock_from_log(last_log, khz)
        if args.trace_out:
            from persistent_tiled_gemm_amd.trace import write_chrome_trace
            n = write_chrome_trace(last_log, khz, args.trace_out, label="8192^3",
                                   metadata={"workload": "square_8192", "sched": args.mode})
            log(f"wrote {n} tile events to {args.trace_out}")

    modes = {}
    if not args.no_modes:
        other = dict(fields, claim_policy=1 - args.claim_policy)
        plan_other = ptg.gemm_create(**other)
        plan_group = ptg.gemm_create(**dict(fields, claim_group=4, raster=1, raster_group=2))
        # the dynamic grid stopping at the resident workgroups instead of one launch slot per tile
        plan_resident = ptg.gemm_create(**dict(fields, dynamic_grid=ptg.GRID_RESIDENT))
        runs = [("nonpersistent", "nonpersistent", plan), ("static", "static", plan), ("dynamic", "dynamic", plan),
                ("dynamic_single_counter" if args.claim_policy == 1 else "dynamic_xcd_counters", "dynamic", plan_other),
                ("dynamic_claim_groups_2x2", "dynamic", plan_group),
                ("dynamic_resident_grid", "dynamic", plan_resident)]
        fns = {name: (lambda mode=mode, pl=pl: ptg.gemm_run(A, B, C, pl, mode=mode, stream=stream))
               for name, mode, pl in runs}
        # the same product with B given as N x K (plan b_layout 1: C = A . Bt^T)
        plan_bt = ptg.gemm_create(**dict(fields, b_layout=1))
        Bt = B.t().contiguous()
        fns["dynamic_b_transposed"] = lambda: ptg.gemm_run(A, Bt, C, plan_bt, mode="dynamic", stream=stream)
        # context only: the vendor library's bf16 GEMM at the same shape (torch.matmul -> hipBLASLt), which
        # writes a bf16 C (half of our fp32 C bytes), and, where torch offers it, the same product with an
        # fp32 C (torch.mm with out_dtype), the exact counterpart of this kernel
        fns["vendor_matmul_bf16_out"] = lambda: torch.matmul(A, B)
        try:
            torch.mm(A, B, out_dtype=torch.float32)
            torch.cuda.synchronize()
            fns["vendor_mm_fp32_out"] = lambda: torch.mm(A, B, out_dtype=torch.float32)
        except Exception as e:  # not offered by the installed torch: reported as absent (context only)
            log(f"vendor fp32-output mm unavailable: {e}")
        # the clock drifts over tens of milliseconds under this load, so the variants are timed in
        # interleaved blocks (alternating order), not one after another
        per_mode = time_interleaved(fns, rounds=4, per_round=max(5, args.steps // 5), stream=stream)
        for name, m_ms in per_mode.items():
            modes[name] = {"ms": m_ms, "tflops": flops / (m_ms * 1e-3) / 1e12,
                           "frac_peak": flops / (m_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        for name, mode, pl in runs:
            # the log holds the last run: three back to back, so that it is not a first launch after a pause
            for _ in range(3):
                ptg.gemm_run(A, B, C, pl, mode=mode, stream=stream)
            mk = makespan_from_log(ptg.gemm_read_log(pl), khz) if not args.no_log else None
            if mk:
                modes[name].update(makespan_us=mk["makespan_us"], tile_median_us=mk["tile_median_us"])
        plan_other.destroy()
        plan_group.destroy()
        plan_resident.destroy()
        plan_bt.destroy()
        del Bt

    roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(1.0),
            "kernel": f"ptg_gemm_kernel<256,256,{args.mode}>", "avg_launch_ms": ms,
            "algorithmic_flop_per_launch": flops}
    if clock_ghz:
        # the dense bf16 rate at the clock the GEMM itself ran at (256 CUs x 4096 flop per clock)
        peak_at_clock = info["cu_count"] * 4096 * clock_ghz * 1e-3
        roof.update(clock_ghz=clock_ghz, peak_at_clock=peak_at_clock, frac_at_clock=tflops / peak_at_clock,
                    clock_source="tile log of the last timed launch: s_memtime cycles / s_memrealtime ticks")

    out = {"metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "square_8192", "M": M, "N": N, "K": K, "tile": [256, 256, 32],
                      "sched": args.mode, "claim_policy": "xcd_counters" if args.claim_policy == 1 else "single_counter",
                      "claims_ahead": args.claims_ahead, "ring_depth": 3,
                      "raster_group": args.raster_group, "k_order": "auto (8192^3: one phase per XCD region)",
                      "tile_log": not args.no_log, "accumulate": "fp32",
                      "output": "fp32"},
           "frac_peak": tflops / PEAK_BF16_TFLOPS, "roofline": roof,
           "modes": modes}

    # context for the roofline: the MFMA-only rate and clock with random operands (no memory traffic),
    # the ceiling the power limit leaves any bf16 GEMM on this part
    if not args.no_modes:
        # the kernel's own instruction (16 x 16 x 32) first, then the 32 x 32 x 16 form for comparison
        ptg.gemm_mfma_probe(iters=40000, random_operands=True, mfma_block=16)  # warm-up: the clock settles
        out["mfma_ceiling"] = dict(ptg.gemm_mfma_probe(iters=40000, random_operands=True, mfma_block=16),
                                   what="MFMA-only kernel of v_mfma_f32_16x16x32_bf16 (the 256 x 256 tiles' "
                                        "instruction), random bf16 operands, all CUs, second of two runs")
        out["mfma_ceiling"]["tflops_frac_achieved"] = tflops / out["mfma_ceiling"]["tflops"]
        ptg.gemm_mfma_probe(iters=40000, random_operands=True, mfma_block=32)
        out["mfma_ceiling"]["mfma_32x32x16"] = ptg.gemm_mfma_probe(iters=40000, random_operands=True, mfma_block=32)
        # the memory-side counterpart: what plain streaming kernels reach (1 GiB, four times the last-level
        # cache), the practical ceiling for the HBM-bound tail-boundary shapes below
        out["hbm_ceiling"] = {"read_gbs": ptg.gemm_hbm_probe(1 << 30, "read", reps=20),
                              "copy_gbs": ptg.gemm_hbm_probe(1 << 30, "copy", reps=20),
                              "what": "plain streaming kernels over 1 GiB (16-byte non-temporal loads/stores per lane): "
                                      "read once; copy counts bytes read + written"}
    if not args.no_tail:
        out["tail"] = run_tail_sections(ptg, torch, stream, khz, (p, A, B, C))
        if "hbm_ceiling" in out:
            ceil = out["hbm_ceiling"]["read_gbs"]
            for r in out["tail"]["tail_boundary"].values():
                for v in r.values():
                    if "hbm_gbs" in v:
                        v["frac_of_read_ceiling"] = v["hbm_gbs"] / ceil
    plan.destroy()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(p)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Measured makespans against the discrete-event scheduler model (oracle.sched_model).

Absolute makespans are hardware facts (parity unpinned); what is checked is the
order the pages claim (dynamic finishes before static when slots are unequal or
tile costs uneven) and that each measured makespan, in units of the measured tile
time t, lies within a band around the model fed with the same t (or the fitted
per-tile costs) and the same slot availability. Bands are wide on purpose: the
model ignores launch, claim and memory effects.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from oracle.ownership import split_units
from oracle.sched_model import simulate
from tests.gpu_util import say, torch_mod
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _span(rec, khz):
    ran = rec[rec["visits"] > 0]
    r0 = ran["r0"].astype(np.float64)
    r1 = ran["r1"].astype(np.float64)
    return (r1.max() - r0.min()) / khz * 1e3, np.median(r1 - r0) / khz * 1e3, ran


def test_partial_occupancy_against_model():
    torch = torch_mod()
    p = make_workload("square_8192").problems[0]
    A, B = ptg.bf16_from_bits(p.a_bits), ptg.bf16_from_bits(p.b_bits)
    C = torch.empty((p.M, p.N), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024)
    khz = ptg.gemm_plan_info_get(plan)["wallclock_khz"]
    spoil = torch.cuda.Stream()
    res = {}
    for mode in ("static", "dynamic"):
        say(f"case partial occupancy vs model mode={mode}")
        ptg.gemm_run(A, B, C, plan, mode=mode)
        torch.cuda.synchronize()
        slog = torch.zeros(64 * 4, dtype=torch.int64, device="cuda")
        ptg.gemm_test_spoiler(64, 2_000_000, stream=spoil, log=slog, wait_resident_ms=2000.0)
        ptg.gemm_run(A, B, C, plan, mode=mode)
        torch.cuda.synchronize()
        span, t, ran = _span(ptg.gemm_read_log(plan), khz)
        sl = slog.cpu().numpy().reshape(64, 4).astype(np.float64)
        res[mode] = (span, t, (sl[:, 1].max() - ran["r0"].astype(np.float64).min()) / khz * 1e3)
    # each mode against the model fed with its own measured tile time t: under the
    # spoiler the dynamic run's tiles take 7-25% longer than the static run's (a
    # memory-system effect the model does not describe), so one t for both modes
    # would put that difference on the scheduler
    for mode in ("static", "dynamic"):
        span, t, spoiler_end = res[mode]
        avail = [0.0] * 192 + [max(spoiler_end, 0.0) / t] * 64
        model = simulate([1.0] * 1024, mode, avail=avail, P=256).makespan
        got = span / t
        say(f"  {mode}: measured {got:.2f} t (t = {t:.1f} us), model {model:.2f} t")
        assert 0.8 * model <= got <= 1.25 * model, (mode, got, model)
    assert res["dynamic"][0] < res["static"][0]
    plan.destroy()


def test_grouped_uneven_against_model():
    torch = torch_mod()
    w = make_workload("grouped_uneven")
    As = [ptg.bf16_from_bits(q.a_bits) for q in w.problems]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in w.problems]
    Cs = [torch.empty((q.M, q.N), dtype=torch.float32, device="cuda") for q in w.problems]
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024)
    khz = ptg.gemm_plan_info_get(plan)["wallclock_khz"]
    ks = np.array([q.K for q in w.problems])
    spans = {}
    for mode in ("static", "dynamic"):
        say(f"case grouped vs model mode={mode}")
        for _ in range(2):
            ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=mode)
        torch.cuda.synchronize()
        span, _, ran = _span(ptg.gemm_read_log(plan), khz)
        spans[mode] = span
        if mode == "static":
            dur = (ran["r1"] - ran["r0"]).astype(np.float64) / khz * 1e3
            alpha, beta = np.polyfit(ks[ran["problem"]] / 64.0, dur, 1)
    costs = [alpha * (ks[t // 16] / 64.0) + beta for t in range(1024)]
    for mode in ("static", "dynamic"):
        model = simulate(costs, mode, slots=256, P=256).makespan
        say(f"  {mode}: measured {spans[mode]:.1f} us, model {model:.1f} us")
        assert 0.8 * model <= spans[mode] <= 1.3 * model, (mode, spans[mode], model)
    assert spans["dynamic"] < spans["static"]
    plan.destroy()


def _model_from_log(ran, khz, slots):
    """The dynamic scheduler model fed with the run's own logged unit durations
    (in unit order): the makespan the pages' greedy hand-out gives those costs."""
    order = np.argsort(ran["unit"], kind="stable")
    dur = ((ran["r1"] - ran["r0"]).astype(np.float64) / khz * 1e3)[order]
    return simulate(list(dur), "dynamic", slots=slots).makespan


def test_tail_split_shortens_the_partial_wave():
    """T = 257 tiles on 256 workers. Whole tiles: the last tile starts when the
    first worker frees up. Split: its K-chunks run on idle workers. Each run's
    makespan is checked against the model fed with that run's logged unit
    durations (the lone 257th tile runs faster than a first-wave tile on this
    memory-bound shape, and a split tile's last chunk carries the fix-up: both
    are in the logged durations), and the split run must be shorter."""
    torch = torch_mod()
    q = make_workload("tail_257").problems[0]
    A, B = ptg.bf16_from_bits(q.a_bits), ptg.bf16_from_bits(q.b_bits)
    C = torch.empty((q.M, q.N), dtype=torch.float32, device="cuda")
    whole = ptg.gemm_create(tile_edge=256, log_capacity=512)
    split = ptg.gemm_create(tile_edge=256, log_capacity=512, tail_split=4)
    khz = ptg.gemm_plan_info_get(whole)["wallclock_khz"]
    res = {}
    for name, plan in (("whole", whole), ("split", split)):
        say(f"case tail_257 {name}")
        for _ in range(3):
            ptg.gemm_run(A, B, C, plan, mode="dynamic")
        torch.cuda.synchronize()
        span, t, ran = _span(ptg.gemm_read_log(plan), khz)
        res[name] = (span, t, _model_from_log(ran, khz, 256), ran)
    t = res["whole"][1]
    nk = q.K // 32
    units = split_units(257, 256, nk, 4, min_chunk_steps=8)
    assert len(res["split"][3]) == len(units)
    lone = res["whole"][3][res["whole"][3]["unit"] == 256]
    lone_us = float((lone["r1"] - lone["r0"]).astype(np.float64)[0] / khz * 1e3)
    for name in ("whole", "split"):
        span, _, model, _ = res[name]
        say(f"  {name}: measured {span:.1f} us = {span / t:.2f} t, model on the logged durations {model:.1f} us "
            f"(t = {t:.1f} us, lone 257th tile {lone_us:.1f} us)")
        assert 0.9 * model <= span <= 1.12 * model, (name, span, model)
    assert res["split"][0] < 0.95 * res["whole"][0]
    whole.destroy()
    split.destroy()


def test_grouped_longest_k_first_against_model():
    torch = torch_mod()
    w = make_workload("grouped_uneven")
    As = [ptg.bf16_from_bits(q.a_bits) for q in w.problems]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in w.problems]
    Cs = [torch.empty((q.M, q.N), dtype=torch.float32, device="cuda") for q in w.problems]
    ks = np.array([q.K for q in w.problems])
    spans = {}
    for order in (0, 1):
        plan = ptg.gemm_create(tile_edge=256, log_capacity=1024, group_order=order)
        khz = ptg.gemm_plan_info_get(plan)["wallclock_khz"]
        say(f"case grouped claim order {order}")
        for _ in range(3):
            ptg.gemm_run_grouped(As, Bs, Cs, plan, mode="dynamic")
        torch.cuda.synchronize()
        span, _, ran = _span(ptg.gemm_read_log(plan), khz)
        spans[order] = span
        if order == 0:
            dur = (ran["r1"] - ran["r0"]).astype(np.float64) / khz * 1e3
            alpha, beta = np.polyfit(ks[ran["problem"]] / 64.0, dur, 1)
        plan.destroy()
    costs = [alpha * (k / 64.0) + beta for k in ks]
    from oracle.sched_model import lpt_claim_order
    model_given = simulate([costs[t // 16] for t in range(1024)], "dynamic", slots=256).makespan
    model_lpt = simulate([costs[t // 16] for t in lpt_claim_order(costs, [16] * 64)], "dynamic", slots=256).makespan
    say(f"  as given {spans[0]:.1f} us (model {model_given:.1f}), longest K first {spans[1]:.1f} us "
        f"(model {model_lpt:.1f})")
    assert 0.8 * model_lpt <= spans[1] <= 1.3 * model_lpt
    assert spans[1] < spans[0]

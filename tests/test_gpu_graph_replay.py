"""A single GEMM launch captured into a HIP graph and replayed: every replay must
give the eager result bit for bit. A replay re-runs the same kernel arguments on
the same scheduler-state set, so this holds only because each run leaves its
claim counters, gate and split-arrival counts at zero when it ends. Covered for
a plan's gemm_run and for gemm_run_noalloc (the entry point for callers that
cannot allocate, such as code under graph capture), in every mode; between
replays the program runs eager work of its own and synchronises.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import assert_close_rows, check_log, say, torch_mod, upload
from workloads import make_problem

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")


def _replay_and_check(run, C, eager, replays=5):
    torch = torch_mod()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run(s)                    # eager on the capture stream first (plan state, first-call set-up)
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        run(s)
    other = torch.randn(512, 512, device="cuda")
    for i in range(replays):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), f"replay {i} differs from the eager run"
        other = other @ other.T / 512.0   # the program's own eager work between replays
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("mode", MODES)
def test_plan_run_replayed_from_a_graph(mode):
    torch = torch_mod()
    p = make_problem(2048, 1536, 1024, "normal", seed=80)   # 48 tiles
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256)
    ptg.gemm_run(A, B, C, plan, mode=mode)
    ptg.gemm_sync(plan)
    eager = C.clone()
    assert_close_rows(p, eager.cpu().numpy(), [0, 255, 1024, 2047])
    say(f"case graph replay gemm_run mode={mode}")
    _replay_and_check(lambda s: ptg.gemm_run(A, B, C, plan, mode=mode, stream=s), C, eager)
    assert ptg.gemm_sync(plan, strict=False) == 0
    plan.destroy()


@pytest.mark.parametrize("mode", MODES)
def test_noalloc_run_replayed_from_a_graph(mode):
    torch = torch_mod()
    p = make_problem(1536, 2048, 512, "uniform", seed=81)
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ptg.gemm_run_noalloc(A, B, C, mode=mode, status=status)
    torch.cuda.synchronize()
    eager = C.clone()
    assert_close_rows(p, eager.cpu().numpy(), [0, 700, 1535])
    say(f"case graph replay gemm_run_noalloc mode={mode}")
    _replay_and_check(lambda s: ptg.gemm_run_noalloc(A, B, C, mode=mode, status=status, stream=s), C, eager)
    assert int(status.item()) == 0


def test_split_tail_replayed_from_a_graph():
    # the split tiles' arrival counts must be back at zero for the next replay
    torch = torch_mod()
    plan = ptg.gemm_create(tile_edge=256, tail_split=4)
    info = ptg.gemm_plan_info_get(plan)
    T = info["occupancy"] * info["cu_count"] + 2
    p = make_problem(T * 256, 256, 1024, "uniform", seed=82)
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    ptg.gemm_run(A, B, C, plan, mode="dynamic")
    ptg.gemm_sync(plan)
    assert ptg.gemm_plan_info_get(plan)["last_split_chunks"] >= 2
    eager = C.clone()
    rows = list(range((T - 2) * 256, T * 256, 9))
    assert_close_rows(p, eager.cpu().numpy(), rows + [0])
    say("case graph replay split tail")
    _replay_and_check(lambda s: ptg.gemm_run(A, B, C, plan, mode="dynamic", stream=s), C, eager)
    plan.destroy()


@pytest.mark.parametrize("mode,order,policy", [("static", 0, 1), ("dynamic", 0, 1), ("dynamic", 1, 2)])
def test_grouped_run_replayed_from_a_graph(mode, order, policy):
    # the problem table was uploaded by the eager run and is unchanged, so the
    # captured call holds the kernel only; every replay must match the eager run
    torch = torch_mod()
    shapes = [(300, 264, 520), (0, 64, 64), (700, 256, 64), (256, 136, 1000), (1, 8, 8), (513, 704, 96)]
    problems = [make_problem(M, N, K, "uniform", seed=90 + i) for i, (M, N, K) in enumerate(shapes)]
    As = [ptg.bf16_from_bits(q.a_bits) for q in problems]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in problems]
    Cs = [torch.full((q.M, q.N), float("nan"), dtype=torch.float32, device="cuda") for q in problems]
    plan = ptg.gemm_create(tile_edge=256, group_order=order, claim_policy=policy)
    ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=mode)
    ptg.gemm_sync(plan)
    eager = [c.clone() for c in Cs]
    for q, c in zip(problems, eager):
        if q.M:
            assert_close_rows(q, c.cpu().numpy(), [0, q.M - 1])
    say(f"case graph replay grouped mode={mode} group_order={order} claim_policy={policy}")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=mode, stream=s)
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=mode, stream=s)
    other = torch.randn(512, 512, device="cuda")
    for i in range(4):
        for c in Cs:
            c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (c, e) in enumerate(zip(Cs, eager)):
            assert torch.equal(c, e), f"replay {i}: problem {j} differs from the eager run"
        other = other @ other.T / 512.0
        torch.cuda.synchronize()
    del g
    assert ptg.gemm_sync(plan, strict=False) == 0
    plan.destroy()


def test_replays_between_uncaptured_runs():
    # a captured launch runs on the plan's graph state set; uncaptured runs of the
    # same plan alternate between the two other sets and do not clean up after
    # themselves. Replays and uncaptured runs in any order must all give the eager
    # result (every mode, twice over, so that each uncaptured set is reused)
    torch = torch_mod()
    p = make_problem(1800, 1288, 520, "uniform", seed=83)   # 48 tiles, ragged edges and K tail
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024)
    ptg.gemm_run(A, B, C, plan, mode="dynamic")
    ptg.gemm_sync(plan)
    eager = C.clone()
    assert_close_rows(p, eager.cpu().numpy(), [0, 255, 256, 1024, 1799])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ptg.gemm_run(A, B, C, plan, mode="dynamic", stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ptg.gemm_run(A, B, C, plan, mode="dynamic", stream=s)
    for rnd in range(2):
        for mode in MODES:
            say(f"case replay between uncaptured runs round={rnd} mode={mode}")
            C.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(C, eager), f"replay before the {mode} run differs"
            C.fill_(float("nan"))
            ptg.gemm_run(A, B, C, plan, mode=mode)
            ptg.gemm_sync(plan)
            assert torch.equal(C, eager), f"uncaptured {mode} run differs"
            check_log(plan, mode, 48, P=ptg.gemm_plan_info_get(plan)["last_grid"] if mode == "static" else None)
    del g
    assert ptg.gemm_sync(plan, strict=False) == 0
    plan.destroy()

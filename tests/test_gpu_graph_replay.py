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
from tests.gpu_util import assert_close_rows, say, torch_mod, upload
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

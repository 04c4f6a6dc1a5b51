"""GPU parity of the longest-K-first claim order for grouped runs (group_order = 1).

The log's unit -> tile map must equal oracle.sched_model.lpt_claim_order, every
unit runs exactly once under each scheduler's ownership rule, each tile covers
its own problem's K exactly once, and every C_g matches the oracle.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from oracle.sched_model import lpt_claim_order
from tests.gpu_util import assert_close_full, assert_close_rows, check_log, make_plan, say, torch_mod
from workloads import make_problem, make_workload

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")


def _run_grouped(problems, plan, mode):
    torch = torch_mod()
    As = [ptg.bf16_from_bits(q.a_bits) for q in problems]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in problems]
    Cs = [torch.full((q.M, q.N), float("nan"), dtype=torch.float32, device="cuda") for q in problems]
    ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=mode)
    torch.cuda.synchronize()
    return [c.cpu().numpy() for c in Cs]


def _tile_k(problems, tile):
    ks = []
    for q in problems:
        ks += [q.K] * (-(-q.M // tile) * -(-q.N // tile))
    return np.array(ks)


def test_lpt_order_small_ragged_problems():
    shapes = [(300, 264, 520), (128, 520, 1000), (700, 256, 64), (256, 136, 1000), (1, 8, 8)]
    problems = [make_problem(M, N, K, "uniform", seed=i) for i, (M, N, K) in enumerate(shapes)]
    tiles = [-(-M // 256) * -(-N // 256) for M, N, _ in shapes]
    T = sum(tiles)
    plan = make_plan(256, group_order=1)
    want = lpt_claim_order([q.K for q in problems], tiles)
    for mode in MODES:
        say(f"case lpt small mode={mode}")
        cs = _run_grouped(problems, plan, mode)
        for q, c in zip(problems, cs):
            assert_close_full(q, c)
        info = ptg.gemm_plan_info_get(plan)
        log = check_log(plan, mode, T, P=info["last_grid"] if mode == "static" else None,
                        K=_tile_k(problems, 256))
        assert log["tile"].tolist() == want
        starts = np.cumsum([0] + tiles)
        assert np.array_equal(log["problem"], np.searchsorted(starts, log["tile"], side="right") - 1)
    plan.destroy()


def test_lpt_order_grouped_uneven_workload():
    w = make_workload("grouped_uneven")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024, group_order=1)
    want = lpt_claim_order([q.K for q in w.problems], [16] * 64)
    rng = np.random.default_rng(9)
    for mode in MODES:
        say(f"case lpt grouped_uneven mode={mode}")
        cs = _run_grouped(w.problems, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        log = check_log(plan, mode, 1024, P=info["last_grid"] if mode == "static" else None,
                        K=_tile_k(w.problems, 256))
        assert log["tile"].tolist() == want
        for g in range(0, 64, 9):
            rows = sorted(set(rng.integers(0, 1024, size=6).tolist() + [0, 1023]))
            assert_close_rows(w.problems[g], cs[g], rows)
    plan.destroy()

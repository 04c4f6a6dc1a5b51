"""GPU parity of the longest-K-first claim order for grouped runs (group_order = 1).

The log's unit -> tile map must equal oracle.sched_model.lpt_claim_order, every
unit runs exactly once under each scheduler's ownership rule, each tile covers
its own problem's K exactly once, and every C_g matches the oracle. With
contiguous XCD regions (claim_policy = 2) the sorted problems are dealt to the
eight regions in snake order, and the log must show that order instead.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from oracle.sched_model import lpt_claim_order
from tests.gpu_util import GroupedReference, assert_close_full, check_log, make_plan, say, torch_mod
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
    ref = GroupedReference(w.problems, seed=9)
    for mode in MODES:
        say(f"case lpt grouped_uneven mode={mode}")
        cs = _run_grouped(w.problems, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        log = check_log(plan, mode, 1024, P=info["last_grid"] if mode == "static" else None,
                        K=_tile_k(w.problems, 256))
        assert log["tile"].tolist() == want
        ref.check(cs, f"lpt {mode}")      # all 64 problems
    plan.destroy()


def _dealt_order(ks, tiles, regions=8):
    """Tile ids in claim order: problems by descending K (stable), dealt to the
    regions 0..7, 7..0, 0..7, ..., the regions' lists concatenated."""
    order = sorted(range(len(ks)), key=lambda g: -ks[g])
    dealt = [[] for _ in range(regions)]
    for i, g in enumerate(order):
        rnd, pos = divmod(i, regions)
        dealt[pos if rnd % 2 == 0 else regions - 1 - pos].append(g)
    starts = np.cumsum([0] + list(tiles))
    return [t for lst in dealt for g in lst for t in range(starts[g], starts[g + 1])]


def test_lpt_dealt_to_contiguous_regions():
    w = make_workload("grouped_uneven")
    ks = [q.K for q in w.problems]
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1024, group_order=1, claim_policy=2)
    want = _dealt_order(ks, [16] * 64)
    assert sorted(want) == list(range(1024))
    # each region (128 units) holds eight whole problems; with the snake deal the
    # regions' K sums differ by at most max K - min K
    sums = [sum(ks[want[r * 128 + 16 * j] // 16] for j in range(8)) for r in range(8)]
    assert max(sums) - min(sums) <= max(ks) - min(ks)
    ref = GroupedReference(w.problems, seed=11)
    for mode in MODES:
        say(f"case lpt dealt grouped_uneven policy=2 mode={mode}")
        cs = _run_grouped(w.problems, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        log = check_log(plan, mode, 1024, P=info["last_grid"] if mode == "static" else None,
                        K=_tile_k(w.problems, 256))
        assert log["tile"].tolist() == want
        ref.check(cs, f"lpt dealt {mode}")   # all 64 problems
    plan.destroy()


def test_contiguous_regions_small_ragged_problems():
    # 21 tiles over 8 regions (five of 3 ids, three of 2): regions cut through problems
    shapes = [(300, 264, 520), (128, 520, 1000), (700, 256, 64), (256, 136, 1000), (1, 8, 8), (513, 704, 96)]
    problems = [make_problem(M, N, K, "uniform", seed=20 + i) for i, (M, N, K) in enumerate(shapes)]
    tiles = [-(-M // 256) * -(-N // 256) for M, N, _ in shapes]
    T = sum(tiles)
    for order in (0, 1):
        plan = make_plan(256, group_order=order, claim_policy=2)
        want = _dealt_order([q.K for q in problems], tiles) if order == 1 else list(range(T))
        say(f"case contiguous regions small ragged T={T} group_order={order}")
        cs = _run_grouped(problems, plan, "dynamic")
        for q, c in zip(problems, cs):
            assert_close_full(q, c)
        log = check_log(plan, "dynamic", T, K=_tile_k(problems, 256))
        assert log["tile"].tolist() == want
        plan.destroy()


@pytest.mark.parametrize("G", [300, 1100])
@pytest.mark.parametrize("order,policy", [(0, 1), (1, 1), (1, 2)])
def test_many_problems_with_empty_ones(G, order, policy):
    """More problems than one round of the kernel's problem lookup covers (256
    table entries), some of them with no tiles (M or N zero, sharing their first
    unit with the next problem): every unit must find its own problem, in the
    given order, longest K first, and dealt to contiguous regions."""
    rng = np.random.default_rng(G + 10 * order + policy)
    shapes = [(int(rng.choice([0, 1, 40, 136, 264, 300])), int(rng.choice([0, 8, 136, 264])),
               int(rng.choice([8, 64, 136]))) for _ in range(G)]
    problems = [make_problem(M, N, K, "uniform", seed=1000 + i) for i, (M, N, K) in enumerate(shapes)]
    tiles = [-(-M // 256) * -(-N // 256) for M, N, _ in shapes]
    ks = [K for _, _, K in shapes]
    T = sum(tiles)
    assert sum(1 for t in tiles if t == 0) > G // 4 and T > 256
    if order == 0:
        want = list(range(T))
    elif policy == 2:
        want = _dealt_order(ks, tiles)
    else:
        want = lpt_claim_order(ks, tiles)
    plan = make_plan(256, group_order=order, claim_policy=policy, max_groups=2048)
    for mode in MODES:
        say(f"case many problems G={G} T={T} group_order={order} claim_policy={policy} mode={mode}")
        cs = _run_grouped(problems, plan, mode)
        for q, c in zip(problems, cs):
            if q.M and q.N:
                assert_close_full(q, c)
        info = ptg.gemm_plan_info_get(plan)
        log = check_log(plan, mode, T, P=info["last_grid"] if mode == "static" else None, K=_tile_k(problems, 256))
        assert log["tile"].tolist() == want
    plan.destroy()

"""GPU parity of claim groups: one claim (static step, non-persistent block) takes
claim_group consecutive tile ids, run back to back by one worker.

Checked: C against the oracle, every tile exactly once, each unit's tiles on one
worker back to back in id order, the per-mode ownership rules on unit ids, the K
cover of every tile, and numerics bitwise equal to single-tile claims (same tile
code, same k order).
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import assert_close_full, check_log, make_plan, run, say
from workloads import make_problem

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")


@pytest.mark.parametrize("group,raster,policy", [(2, 0, 1), (4, 2, 1), (3, 0, 1), (3, 0, 2), (4, 2, 0)])
def test_claim_groups_all_modes(group, raster, policy):
    # claim policies 1 and 2 spread the units over eight XCD regions (interleaved
    # or contiguous runs of unit ids), policy 0 hands them out from one counter
    M, N, K = 1800, 1288, 200      # 8 x 6 = 48 tiles of 256, ragged M, N and K
    p = make_problem(M, N, K, "uniform", seed=group)
    kw = {"raster": 1, "raster_group": raster} if raster else {}
    plan = make_plan(256, claim_group=group, claim_policy=policy, **kw)
    ref = make_plan(256, **kw)
    T = 48
    for mode in MODES:
        say(f"case claim group={group} raster={raster} policy={policy} mode={mode}")
        c = run(p, plan, mode)
        assert_close_full(p, c)
        info = ptg.gemm_plan_info_get(plan)
        assert info["last_units"] == -(-T // group) and info["last_claim_group"] == group
        check_log(plan, mode, T, P=info["last_grid"] if mode == "static" else None, K=K, group=group)
        assert np.array_equal(c, run(p, ref, mode))
    plan.destroy()
    ref.destroy()


def test_claim_groups_few_static_workers_and_no_split():
    # 15 tiles in units of 4 (the last unit holds 3); tail splitting is off with claim groups
    M, N, K = 1280, 768, 512
    p = make_problem(M, N, K, "normal", seed=5)
    plan = make_plan(256, claim_group=4, static_workers=2, tail_split=8)
    for mode in ("static", "dynamic"):
        say(f"case claim group 4 T=15 mode={mode}")
        c = run(p, plan, mode)
        assert_close_full(p, c)
        info = ptg.gemm_plan_info_get(plan)
        assert info["last_items"] == 15 and info["last_units"] == 4 and info["last_split_chunks"] == 1
        log = check_log(plan, mode, 15, P=2 if mode == "static" else None, K=K, group=4)
        if mode == "static":
            assert sorted(set(log["worker"][log["unit"] % 2 == 0].tolist())) == [0]
    plan.destroy()


def test_claim_groups_ignored_for_grouped_runs():
    torch = __import__("torch")
    probs = [make_problem(300, 264, 128, "uniform", seed=i) for i in range(3)]
    plan = make_plan(256, claim_group=4)
    As = [ptg.bf16_from_bits(q.a_bits) for q in probs]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in probs]
    Cs = [torch.full((q.M, q.N), float("nan"), dtype=torch.float32, device="cuda") for q in probs]
    say("case claim group grouped run")
    ptg.gemm_run_grouped(As, Bs, Cs, plan, mode="dynamic")
    torch.cuda.synchronize()
    for q, c in zip(probs, Cs):
        assert_close_full(q, c.cpu().numpy())
    info = ptg.gemm_plan_info_get(plan)
    assert info["last_claim_group"] == 1 and info["last_units"] == 12
    check_log(plan, "dynamic", 12, K=128)
    plan.destroy()

"""GPU parity of the K order (plan field k_rotation).

A unit may walk its K range from the first k-step or from a rotated start; the
sum is the same and only the fp32 rounding order inside a tile changes. Checked
for every order: C within the acceptance bound against the oracle, bitwise the
same C under every scheduler (the order is a function of the unit id alone),
every unit once and every tile's K range covered once; exact on integer inputs
(where every order must give the closed form bit for bit); the plain order kept
when K has a partial k-step; and the automatic choice the plan reports.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import assert_close_rows, check_log, make_plan, run, say
from workloads import GemmProblem, f32_to_bf16_bits, make_problem

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")
ORDERS = {"off": ptg.KROT_OFF, "xcd": ptg.KROT_XCD, "xcd2": ptg.KROT_XCD2, "unit": ptg.KROT_UNIT}


@pytest.mark.parametrize("order", list(ORDERS))
@pytest.mark.parametrize("shape", [(1000, 776, 512), (2304, 264, 1024), (300, 2056, 96)])
def test_every_k_order_matches_the_oracle_under_every_scheduler(order, shape):
    M, N, K = shape
    p = make_problem(M, N, K, "normal", seed=M + N + K)
    plan = make_plan(256, k_rotation=ORDERS[order])
    tiles = -(-M // 256) * -(-N // 256)
    outs = {}
    for mode in MODES:
        say(f"case k order {order} shape={shape} mode={mode}")
        c = run(p, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        assert info["last_k_rotation"] == ORDERS[order]
        check_log(plan, mode, tiles, P=info["last_grid"] if mode == "static" else None, K=K)
        outs[mode] = c
    assert_close_rows(p, outs["dynamic"], range(M))
    assert np.array_equal(outs["static"], outs["dynamic"])
    assert np.array_equal(outs["nonpersistent"], outs["dynamic"])
    plan.destroy()


def test_every_k_order_is_exact_on_integer_inputs():
    # integer-valued bf16 inputs in [-8, 8] with K * 64 < 2^24: every partial sum is an exactly
    # representable fp32 integer, so every order of the sum gives the closed form bit for bit
    rng = np.random.default_rng(17)
    M, N, K = 776, 520, 2048
    ai = rng.integers(-8, 9, size=(M, K))
    bi = rng.integers(-8, 9, size=(K, N))
    p = GemmProblem(f32_to_bf16_bits(ai.astype(np.float32)), f32_to_bf16_bits(bi.astype(np.float32)))
    exact = (ai @ bi).astype(np.float32)
    for order, code in ORDERS.items():
        plan = make_plan(256, k_rotation=code)
        for mode in MODES:
            say(f"case integer k order {order} mode={mode}")
            assert np.array_equal(run(p, plan, mode), exact)
        plan.destroy()


def test_rotated_orders_differ_from_the_plain_one_only_in_rounding():
    # the same products summed in another order: within a few fp32 ulps of the sum's magnitude
    M, N, K = 512, 512, 4096
    p = make_problem(M, N, K, "normal", seed=23)
    ref = run(p, make_plan(256, k_rotation=ptg.KROT_OFF), "dynamic").astype(np.float64)
    scale = np.abs(ref).max()
    for order in ("xcd", "xcd2", "unit"):
        say(f"case k order {order} against the plain order")
        c = run(p, make_plan(256, k_rotation=ORDERS[order]), "dynamic").astype(np.float64)
        assert np.abs(c - ref).max() <= 256 * np.finfo(np.float32).eps * scale
        assert not np.array_equal(c, ref)   # the order did change


def test_partial_k_step_keeps_the_plain_order():
    # K = 520 is not a multiple of 32: every order falls back to the plain one (bitwise)
    p = make_problem(700, 1032, 520, "uniform", seed=29)
    outs = []
    for order, code in ORDERS.items():
        say(f"case K tail k order {order}")
        outs.append(run(p, make_plan(256, k_rotation=code), "dynamic"))
    for c in outs[1:]:
        assert np.array_equal(c, outs[0])
    assert_close_rows(p, outs[0], [0, 255, 256, 699])


def test_k_orders_with_a_split_tail():
    # T = workers + 3 tiles with the tail split into K-chunks: each chunk rotates within its own range
    for order in ("xcd", "xcd2", "unit"):
        plan = make_plan(256, tail_split=4, log_capacity=4096, k_rotation=ORDERS[order])
        info = ptg.gemm_plan_info_get(plan)
        T = info["occupancy"] * info["cu_count"] + 3
        M, N, K = T * 256, 256, 1024
        p = make_problem(M, N, K, "uniform", seed=31)
        say(f"case split tail k order {order} T={T}")
        c = run(p, plan, "dynamic")
        info = ptg.gemm_plan_info_get(plan)
        assert info["last_split_chunks"] >= 2
        check_log(plan, "dynamic", info["last_items"], K=K, tiles=T)
        rows = list(range((T - 3) * 256, M, 5)) + [0, 255, M // 2]
        assert_close_rows(p, c, rows)
        plan.destroy()


def test_automatic_k_order():
    # at most 8 tile columns: two phases per XCD region; more: one; grouped runs: a phase per problem
    import torch
    plan = make_plan(256)
    assert plan.desc.k_rotation == ptg.KROT_AUTO
    for (M, N, K), want in (((512, 2048, 256), ptg.KROT_XCD2), ((512, 2304, 256), ptg.KROT_XCD),
                            ((4096, 256, 512), ptg.KROT_XCD2)):
        p = make_problem(M, N, K, "uniform", seed=N)
        say(f"case auto k order shape={(M, N, K)}")
        c = run(p, plan, "dynamic")
        assert ptg.gemm_plan_info_get(plan)["last_k_rotation"] == want
        assert_close_rows(p, c, [0, M - 1])
    q = make_problem(512, 2304, 256, "uniform", seed=1)
    A, B = ptg.bf16_from_bits(q.a_bits), ptg.bf16_from_bits(q.b_bits)
    C = torch.empty((q.M, q.N), dtype=torch.float32, device="cuda")
    ptg.gemm_run_grouped([A, A], [B, B], [C, C.clone()], plan, mode="dynamic")
    torch.cuda.synchronize()
    assert ptg.gemm_plan_info_get(plan)["last_k_rotation"] == ptg.KROT_UNIT   # a phase per problem
    plan.destroy()


@pytest.mark.parametrize("order", list(ORDERS))
def test_every_k_order_in_grouped_runs(order):
    # grouped runs key the phase to the problem: every order matches the oracle on ragged problems and
    # gives bitwise the same C under every scheduler
    import torch
    shapes = [(300, 264, 512), (520, 776, 1024), (256, 256, 96), (700, 520, 2048), (64, 1032, 256)]
    problems = [make_problem(M, N, K, "normal", seed=90 + i) for i, (M, N, K) in enumerate(shapes)]
    As = [ptg.bf16_from_bits(q.a_bits) for q in problems]
    Bs = [ptg.bf16_from_bits(q.b_bits) for q in problems]
    plan = make_plan(256, k_rotation=ORDERS[order], group_order=1, claim_policy=2)
    T = sum(-(-M // 256) * -(-N // 256) for M, N, _ in shapes)
    outs = {}
    for mode in MODES:
        say(f"case grouped k order {order} mode={mode}")
        Cs = [torch.full((q.M, q.N), float("nan"), dtype=torch.float32, device="cuda") for q in problems]
        ptg.gemm_run_grouped(As, Bs, Cs, plan, mode=mode)
        torch.cuda.synchronize()
        info = ptg.gemm_plan_info_get(plan)
        assert info["last_k_rotation"] == ORDERS[order]
        check_log(plan, mode, T, P=info["last_grid"] if mode == "static" else None)
        outs[mode] = [c.cpu().numpy() for c in Cs]
    for q, c in zip(problems, outs["dynamic"]):
        assert_close_rows(q, c, range(q.M))
    for g in range(len(problems)):
        assert np.array_equal(outs["static"][g], outs["dynamic"][g])
        assert np.array_equal(outs["nonpersistent"][g], outs["dynamic"][g])
    plan.destroy()

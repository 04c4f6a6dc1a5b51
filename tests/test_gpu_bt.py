"""GPU parity of the B^T form (plan b_layout = 1: B given as N x K row-major, C = A . B^T).

The oracle is the plain definition on the same bits: C = A . (B^T)^T in float64
(gemm_ref of A and the transpose of the N x K operand). The B^T kernel reads its
operand from a K-contiguous layout but feeds the MFMAs the same values in the
same k order as the K x N kernel, so for the same logical B both forms must
agree bit for bit; the tile log must be exactly-once in every mode.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import assert_close_full, check_log, make_plan, new_c, say, torch_mod
from oracle.gemm_ref import check_result, decode_bf16, gemm_ref_rows
from workloads import GemmProblem, make_problem, make_workload

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")


def _run(A, B, M, N, plan, mode):
    torch = torch_mod()
    C = new_c(M, N)
    ptg.gemm_run(A, B, C, plan, mode=mode)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("shape", [(384, 512, 512), (1000, 776, 264), (513, 264, 72), (1, 8, 8), (700, 1032, 1240)])
def test_bt_small_shapes_all_modes(tile, shape):
    M, N, K = shape
    p = make_problem(M, N, K, "uniform", seed=M + 2 * N + K)
    bt_bits = np.ascontiguousarray(p.b_bits.T)            # N x K
    A = ptg.bf16_from_bits(p.a_bits)
    Bt = ptg.bf16_from_bits(bt_bits)
    B = ptg.bf16_from_bits(p.b_bits)
    plan_t = make_plan(tile, b_layout=1)
    plan_n = make_plan(tile)
    T = -(-M // tile) * -(-N // tile)
    for mode in MODES:
        say(f"case bt tile={tile} shape={shape} mode={mode}")
        ct = _run(A, Bt, M, N, plan_t, mode).cpu().numpy()
        assert_close_full(GemmProblem(p.a_bits, p.b_bits), ct)
        info = ptg.gemm_plan_info_get(plan_t)
        check_log(plan_t, mode, T, P=info["last_grid"] if mode == "static" else None, K=K)
        cn = _run(A, B, M, N, plan_n, mode).cpu().numpy()
        assert np.array_equal(ct, cn)
    plan_t.destroy()
    plan_n.destroy()


def test_bt_square_8192_sampled_rows():
    torch = torch_mod()
    p = make_workload("square_8192").problems[0]
    A = ptg.bf16_from_bits(p.a_bits)
    B = ptg.bf16_from_bits(p.b_bits)
    Bt = B.t().contiguous()
    plan_t = ptg.gemm_create(tile_edge=256, log_capacity=1024, b_layout=1)
    plan_n = ptg.gemm_create(tile_edge=256, log_capacity=1024)
    rows = np.sort(np.random.default_rng(4).choice(p.M, 48, replace=False))
    idx = torch.as_tensor(rows, device="cuda")
    say("case bt square_8192 dynamic")
    C = torch.empty((p.M, p.N), dtype=torch.float32, device="cuda")
    ptg.gemm_run(A, Bt, C, plan_t, mode="dynamic")
    torch.cuda.synchronize()
    check_log(plan_t, "dynamic", 1024)
    ct = C[idx].cpu().numpy()
    ref = gemm_ref_rows(p.a_bits, p.b_bits, rows)
    rep = check_result(ct, ref, p.K, float(np.abs(decode_bf16(p.a_bits)).max()),
                       float(np.abs(decode_bf16(p.b_bits)).max()))
    assert rep["ok"], rep
    ptg.gemm_run(A, B, C, plan_n, mode="dynamic")
    torch.cuda.synchronize()
    assert np.array_equal(ct, C[idx].cpu().numpy())
    plan_t.destroy()
    plan_n.destroy()


def test_bt_grouped_ragged():
    torch = torch_mod()
    shapes = [(300, 264, 520), (128, 520, 1000), (700, 256, 64), (1, 8, 8)]
    problems = [make_problem(M, N, K, "uniform", seed=i + 40) for i, (M, N, K) in enumerate(shapes)]
    As = [ptg.bf16_from_bits(q.a_bits) for q in problems]
    Bts = [ptg.bf16_from_bits(np.ascontiguousarray(q.b_bits.T)) for q in problems]
    plan = make_plan(256, b_layout=1)
    for mode in MODES:
        say(f"case bt grouped mode={mode}")
        Cs = [new_c(q.M, q.N) for q in problems]
        ptg.gemm_run_grouped(As, Bts, Cs, plan, mode=mode)
        torch.cuda.synchronize()
        for q, c in zip(problems, Cs):
            assert_close_full(q, c.cpu().numpy())
    plan.destroy()


def test_bt_operand_shapes_checked():
    torch = torch_mod()
    plan = make_plan(256, b_layout=1)
    A = torch.zeros((16, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ptg.gemm_run(A, torch.zeros((24, 16), dtype=torch.bfloat16, device="cuda"), new_c(16, 16), plan)  # K x N given
    # K == 0: C is all zeros in every mode
    for mode in MODES:
        C = new_c(300, 264)
        ptg.gemm_run(torch.zeros((300, 0), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((264, 0), dtype=torch.bfloat16, device="cuda"), C, plan, mode=mode)
        torch.cuda.synchronize()
        assert torch.count_nonzero(C).item() == 0 and not torch.isnan(C).any().item()
    plan.destroy()
    with pytest.raises(ptg.PtgError):
        ptg.gemm_create(tile_edge=256, b_layout=2)

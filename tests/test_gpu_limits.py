"""GPU parity at the size limits the C ABI accepts (K up to 2^20, N up to 2^22,
tile counts past 2^16), on sampled elements the oracle computes one by one.

Inputs come from torch's seeded normal generator on the device (not from the
library); their exact bf16 bits are copied back for the oracle.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from oracle.gemm_ref import check_result, decode_bf16, gemm_ref_elements
from tests.gpu_util import check_log, say, torch_mod

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch_mod().int16).cpu().numpy().view(np.uint16)


def _randn(rows, cols, seed, scale):
    torch = torch_mod()
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(rows, cols, device="cuda", generator=g) * scale).to(torch.bfloat16)


def _check_sampled(A, B, C, K, n=48, seed=0):
    torch = torch_mod()
    M, N = C.shape
    rng = np.random.default_rng(seed)
    rows = np.r_[0, M - 1, rng.integers(0, M, size=n)]
    cols = np.r_[N - 1, 0, rng.integers(0, N, size=n)]
    ur, uc = np.unique(rows), np.unique(cols)
    a_bits = _bits(A[torch.as_tensor(ur, device="cuda")])
    b_bits = _bits(B[:, torch.as_tensor(uc, device="cuda")].contiguous())
    ri = np.searchsorted(ur, rows)
    ci = np.searchsorted(uc, cols)
    ref = gemm_ref_elements(a_bits, b_bits, ri, ci)
    got = C[torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")].cpu().numpy()
    # max|a|, max|b| over the whole matrices (the acceptance bound's definition)
    amax = float(A.float().abs().max().item())
    bmax = float(B.float().abs().max().item())
    rep = check_result(got, ref, K, amax, bmax)
    assert rep["ok"], rep


def test_largest_k():
    torch = torch_mod()
    M, N, K = 256, 512, 1 << 20          # one row of two tiles, 16384 k-steps each
    A = _randn(M, K, 1, K ** -0.5)
    B = _randn(K, N, 2, 1.0)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=16)
    for mode in ("static", "dynamic"):
        say(f"case K=2^20 mode={mode}")
        C.fill_(float("nan"))
        ptg.gemm_run(A, B, C, plan, mode=mode)
        torch.cuda.synchronize()
        assert not torch.isnan(C).any().item()
        _check_sampled(A, B, C, K, seed=3)
        info = ptg.gemm_plan_info_get(plan)
        check_log(plan, mode, 2, P=info["last_grid"] if mode == "static" else None, K=K)
    plan.destroy()


def test_largest_n():
    torch = torch_mod()
    M, N, K = 24, 1 << 22, 24             # 16384 tiles of 256, ragged in M and K
    A = _randn(M, K, 3, 1.0)
    B = _randn(K, N, 4, 1.0)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=16384)
    for mode in ("nonpersistent", "dynamic"):
        say(f"case N=2^22 mode={mode}")
        C.fill_(float("nan"))
        ptg.gemm_run(A, B, C, plan, mode=mode)
        torch.cuda.synchronize()
        assert not torch.isnan(C).any().item()
        _check_sampled(A, B, C, K, seed=4)
        check_log(plan, mode, 16384, K=K)
    plan.destroy()


def test_tile_count_past_two_to_the_sixteen():
    torch = torch_mod()
    M, N, K = (1 << 16) * 256, 8, 8      # 65536 tiles, one column of them
    A = _randn(M, K, 5, 1.0)
    B = _randn(K, N, 6, 1.0)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=1 << 16)
    for mode in ("nonpersistent", "static", "dynamic"):
        say(f"case 65536 tiles mode={mode}")
        C.fill_(float("nan"))
        ptg.gemm_run(A, B, C, plan, mode=mode)
        torch.cuda.synchronize()
        assert not torch.isnan(C).any().item()
        _check_sampled(A, B, C, K, seed=5)
        info = ptg.gemm_plan_info_get(plan)
        check_log(plan, mode, 1 << 16, P=info["last_grid"] if mode == "static" else None)
    plan.destroy()


def test_sizes_past_the_limits_are_refused():
    torch = torch_mod()
    plan = ptg.gemm_create(tile_edge=256)
    buf = torch.empty(64, dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    assert ptg.gemm_run_raw(p, p, p, 8, 8, (1 << 20) + 8, plan) == -2
    assert ptg.gemm_run_raw(p, p, p, 8, (1 << 22) + 8, 8, plan) == -2
    assert ptg.gemm_run_raw(p, p, p, (1 << 30) + 1, 8, 8, plan) == -2
    plan.destroy()

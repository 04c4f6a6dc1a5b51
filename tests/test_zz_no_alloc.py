"""gemm_run_noalloc (the entry point for callers that cannot allocate) against
gemm_run with the default 256 x 256 plan: the same kernel and configuration, so
C must be bitwise identical. Two calls in a row per mode, the second with a
smaller (ragged) input, so the second call runs on the scheduler state the
first one left behind; a status word is passed and must stay clear.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import assert_close_rows, say, torch_mod, upload
from workloads import make_problem

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")
SHAPES = [(2048, 1536, 1000), (700, 264, 520)]   # 48 tiles, then 3 ragged tiles


@pytest.mark.parametrize("mode", MODES)
def test_noalloc_matches_gemm_run(mode):
    torch = torch_mod()
    plan = ptg.gemm_create(tile_edge=256)   # the default plan: log off
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, (M, N, K) in enumerate(SHAPES):
        p = make_problem(M, N, K, "normal", seed=60 + i)
        A, B = upload(p)
        want = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        say(f"case noalloc mode={mode} call={i} shape={(M, N, K)}")
        ptg.gemm_run(A, B, want, plan, mode=mode)
        ptg.gemm_sync(plan)
        ptg.gemm_run_noalloc(A, B, got, mode=mode, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        w, g = want.cpu().numpy(), got.cpu().numpy()
        assert not np.isnan(g).any()
        assert np.array_equal(w, g)
        assert_close_rows(p, g, [0, 1, M // 2, M - 1])
    plan.destroy()


def test_noalloc_back_to_back_without_sync():
    """Calls enqueued back to back on one stream (no host synchronisation):
    each run clears the next run's control set, so every call is complete."""
    torch = torch_mod()
    p = make_problem(1024, 1024, 512, "uniform", seed=70)
    A, B = upload(p)
    Cs = [torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(6)]
    say("case noalloc back to back x6")
    for i, C in enumerate(Cs):
        ptg.gemm_run_noalloc(A, B, C, mode=MODES[i % 3])
    torch.cuda.synchronize()
    first = Cs[0].cpu().numpy()
    assert not np.isnan(first).any()
    for C in Cs[1:]:
        assert np.array_equal(C.cpu().numpy(), first)
    assert_close_rows(p, first, [0, 511, 1023])


def test_noalloc_refuses_bad_arguments():
    torch = torch_mod()
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    lib = ptg.load_library()
    import ctypes
    vp = ctypes.c_void_p
    p = buf.data_ptr()
    assert lib.gemm_run_noalloc(vp(p), vp(p), vp(p), 8, 8, (1 << 20) + 8, 2, None, None) == -2
    assert lib.gemm_run_noalloc(vp(p), vp(p), vp(p), 8, 12, 8, 2, None, None) == -2
    assert lib.gemm_run_noalloc(vp(p), vp(p), vp(p + 4), 8, 8, 8, 2, None, None) == -1
    assert lib.gemm_run_noalloc(vp(p), vp(p), vp(p), 8, 8, 8, 2, vp(p + 2), None) == -1

"""GPU tests of the C-ABI boundary: device failures are observable with the tile
log off, runs of one plan on two streams are ordered, and a CU-masked stream
confines the kernel to the compute units it names.

Failure forcing follows the blog post "CUTLASS Cluster Launch Control dynamic
persistent kernel", section "cluster granularity and exit after failure": a
worker that cannot get work must stop, and the failure must be seen. The gate
timeout is forced from the host (every gate slot preset as taken, a short spin
bound), so every workgroup's bounded wait ends and every kernel exits normally.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import assert_close_full, check_log, make_plan, say, torch_mod, upload
from workloads import make_problem

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")
GEMM_E_TIMEOUT = -7


def _problem():
    # 3 x 4 tiles of 256, ragged in M, N and K
    return make_problem(700, 1000, 520, "uniform", seed=41)


@pytest.mark.parametrize("mode", MODES)
def test_gate_timeout_is_reported_with_the_log_off(mode):
    torch = torch_mod()
    p = _problem()
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    # a gate no grid here fills (max_concurrent >= grid), a short spin bound, log off
    plan = ptg.gemm_create(tile_edge=256, log_capacity=0, max_concurrent=1024, gate_spin_limit=64)
    say(f"case gate timeout forced, log off, mode={mode}")
    ptg.gemm_test_preset_gate(plan, 1024)           # every slot taken: every wait runs out
    ptg.gemm_run(A, B, C, plan, mode=mode)
    st = ptg.gemm_sync(plan, strict=False)
    assert st == GEMM_E_TIMEOUT, st
    assert "concurrency gate" in ptg.gemm_last_hip_error(plan)
    assert torch.isnan(C).all().item()              # nobody computed anything
    assert ptg.gemm_sync(plan, strict=False) == 0   # read once, then cleared
    say(f"case gate normal run after the forced one, mode={mode}")
    ptg.gemm_run(A, B, C, plan, mode=mode)          # the preset applied to one run only
    assert ptg.gemm_sync(plan, strict=False) == 0
    assert_close_full(p, C.cpu().numpy())
    plan.destroy()


def test_device_status_is_sticky_across_runs():
    """A failed run followed by a good one: the failure is still reported (by
    gemm_read_log as by gemm_sync), and the good run's log and C are intact."""
    torch = torch_mod()
    p = _problem()
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ptg.gemm_create(tile_edge=256, log_capacity=64, max_concurrent=1024, gate_spin_limit=64)
    say("case sticky status: forced static timeout, then a good dynamic run")
    ptg.gemm_test_preset_gate(plan, 1024)
    ptg.gemm_run(A, B, C, plan, mode="static")
    ptg.gemm_run(A, B, C, plan, mode="dynamic")
    st, rec = ptg.gemm_read_log_status(plan)
    assert st == GEMM_E_TIMEOUT, st
    assert len(rec) == 12 and np.all(rec["visits"] == 1)   # the log is the good run's
    assert_close_full(p, C.cpu().numpy())
    assert ptg.gemm_sync(plan, strict=False) == 0
    with pytest.raises(ptg.PtgError):
        ptg.gemm_test_preset_gate(plan, 1024)
        ptg.gemm_run(A, B, C, plan, mode="nonpersistent")
        ptg.gemm_read_log(plan)                             # strict: raises on the device status
    plan.destroy()


def test_runs_on_two_streams_are_ordered():
    """Back-to-back runs of one plan on two streams, no host synchronisation in
    between: the second run waits for the first on the device, so the scheduler
    state they share is never used by both at once."""
    torch = torch_mod()
    p = make_problem(4096, 2048, 1024, "normal", seed=43)
    q = make_problem(2048, 4096, 512, "normal", seed=44)
    A1, B1 = upload(p)
    A2, B2 = upload(q)
    C1 = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    C2 = torch.full((q.M, q.N), float("nan"), dtype=torch.float32, device="cuda")
    plan = make_plan(256, log_capacity=256)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rnd in range(3):
        say(f"case two streams round {rnd}")
        ptg.gemm_run(A1, B1, C1, plan, mode="dynamic", stream=s1)
        ptg.gemm_run(A2, B2, C2, plan, mode="dynamic", stream=s2)
        check_log(plan, "dynamic", 128)             # the second run's log, synchronised on s2
        s1.synchronize()
        assert not torch.isnan(C1).any().item() and not torch.isnan(C2).any().item()
    from tests.gpu_util import assert_close_rows
    assert_close_rows(p, C1.cpu().numpy(), [0, 255, 256, 2047, 4095])
    assert_close_rows(q, C2.cpu().numpy(), [0, 255, 1024, 2047])
    plan.destroy()


def _cu_key(hw_id, xcc_id):
    return (np.asarray(xcc_id, np.int64) << 8) | ((np.asarray(hw_id, np.int64) >> 8) & 0xFF)


@pytest.mark.parametrize("mode", ("static", "dynamic"))
def test_cu_masked_stream_confines_the_kernel(mode):
    """Half of the compute units in the mask, spread so that every XCD keeps some
    whichever way the mask's bits map to XCDs (eight of every sixteen bits): the
    log shows at most that many distinct CUs, and C is exact."""
    torch = torch_mod()
    info = ptg.gemm_plan_info_get(ptg.gemm_create(tile_edge=256))
    cus = info["cu_count"]
    assert cus % 32 == 0, cus
    words = [0x00FF00FF] * (cus // 32)
    allowed = sum(bin(w).count("1") for w in words)
    p = make_problem(4096, 4096, 512, "uniform", seed=45)   # 256 tiles
    A, B = upload(p)
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    plan = make_plan(256, log_capacity=256)
    stream = ptg.gemm_test_stream_cu_mask(words)
    say(f"case CU-masked stream ({allowed} of {cus} CUs), mode={mode}")
    try:
        ptg.gemm_run(A, B, C, plan, mode=mode, stream=stream.torch_stream)
        info = ptg.gemm_plan_info_get(plan)
        log = check_log(plan, mode, 256, P=info["last_grid"] if mode == "static" else None)
        used = np.unique(_cu_key(log["hw_id"], log["xcc_id"]))
        say(f"  distinct CUs used: {len(used)}; XCDs: {sorted(set((used >> 8).tolist()))}")
        assert 0 < len(used) <= allowed
        assert_close_full(p, C.cpu().numpy())
    finally:
        plan.destroy()        # synchronises the plan's last stream, the masked one, while it is still valid
        stream.destroy()


def test_cu_mask_arguments_are_checked():
    torch = torch_mod()
    cus = ptg.gemm_plan_info_get(ptg.gemm_create(tile_edge=256))["cu_count"]
    for words in ([0], [0xFFFFFFFF] * (cus // 32) + [1]):   # no unit; a unit past the last CU
        with pytest.raises(ptg.PtgError) as e:
            ptg.gemm_test_stream_cu_mask(words)
        assert e.value.status == -1

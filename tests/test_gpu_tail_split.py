"""GPU parity of tail splitting: the tiles of a partial last wave run as K-chunks.

Checked against the oracle: C within the stated bf16/fp32 tolerance (whole and
split tiles alike), the work units the log shows equal oracle.ownership.split_units
(unit id -> tile and K range), every unit ran exactly once under each scheduler's
ownership rule, the units of each tile cover its K range exactly once, and the
split result is deterministic (fixed chunk order of the fix-up sum): bitwise equal
across runs and across schedulers.
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from oracle.ownership import split_units
from tests.gpu_util import assert_close_rows, check_log, make_plan, run, say
from workloads import make_problem

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")


def _expect_units(plan, log, T, workers, K, max_chunks):
    nk = -(-K // 32)                       # 32-deep k-steps; chunks get at least 8 of them
    want = split_units(T, workers, nk, max_chunks, min_chunk_steps=8)
    assert len(log) == len(want), (len(log), len(want))
    tiles = np.array([u[0] for u in want])
    kb = np.minimum(np.array([u[1] for u in want]) * 32, K)
    ke = np.minimum(np.array([u[2] for u in want]) * 32, K)
    assert np.array_equal(log["tile"], tiles)
    assert np.array_equal(log["k_begin"], kb) and np.array_equal(log["k_end"], ke)
    return want


def _split_rows(want, tile_m, M, tiles_n):
    """Every 7th row of the row blocks that hold split tiles."""
    counts = np.bincount([u[0] for u in want])
    rows = set()
    for t in np.nonzero(counts > 1)[0].tolist():
        mt = t // tiles_n
        rows.update(range(mt * tile_m, min(M, (mt + 1) * tile_m), 7))
    return sorted(rows)


@pytest.mark.parametrize("shape", [(257 * 256, 256, 1024), (257 * 256 - 100, 264, 1000)])
def test_tail_split_full_wave_plus_tail(shape):
    M, N, K = shape
    p = make_problem(M, N, K, "uniform", seed=K)
    plan = make_plan(256, tail_split=8, log_capacity=4096)
    info = ptg.gemm_plan_info_get(plan)
    workers = info["occupancy"] * info["cu_count"]
    tn = -(-N // 256)
    T = -(-M // 256) * tn
    outs = {}
    for mode in MODES:
        say(f"case tail split shape={shape} mode={mode}")
        c = run(p, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        U = info["last_items"]
        assert info["last_tiles"] == T and info["last_split_chunks"] >= 2, info
        log = check_log(plan, mode, U, P=info["last_grid"] if mode == "static" else None, K=K, tiles=T)
        want = _expect_units(plan, log, T, workers, K, 8)
        # every row of the split tiles, a sample of the whole ones
        rows = _split_rows(want, 256, M, tn) + [0, 1, 255, 256, M // 2, M - 1]
        assert_close_rows(p, c, rows)
        outs[mode] = c
    assert np.array_equal(outs["static"], outs["dynamic"])
    assert np.array_equal(outs["nonpersistent"], outs["dynamic"])
    c2 = run(p, plan, "dynamic")
    assert np.array_equal(c2, outs["dynamic"])
    plan.destroy()


def test_tail_split_static_few_workers_ragged():
    # P = 5 static workers, 12 tiles: 10 whole, the 2 tail tiles in 2 chunks each;
    # K = 520 is not a multiple of 32 (the last chunk holds the K tail)
    M, N, K = 700, 1024, 520
    p = make_problem(M, N, K, "normal", seed=3)
    plan = make_plan(256, tail_split=8, static_workers=5)
    say("case tail split static P=5")
    c = run(p, plan, "static")
    info = ptg.gemm_plan_info_get(plan)
    T = 3 * 4
    assert info["last_items"] == info["last_units"] == 10 + 2 * 2
    log = check_log(plan, "static", info["last_items"], P=5, K=K, tiles=T)
    _expect_units(plan, log, T, 5, K, 8)
    for w in range(5):
        assert sorted(log["unit"][log["worker"] == w].tolist()) == list(range(w, 14, 5))
    assert_close_rows(p, c, range(M))
    plan.destroy()


def test_tail_split_falls_back_to_whole_tiles():
    # K = 192 is 6 k-steps of 32: fewer than two chunks of 8, so nothing is split
    M, N, K = 257 * 128, 128, 192
    p = make_problem(M, N, K, "uniform", seed=11)
    plan = make_plan(128, tail_split=8, min_lds_bytes=96 * 1024)
    say("case tail split fallback")
    c = run(p, plan, "dynamic")
    info = ptg.gemm_plan_info_get(plan)
    assert info["last_items"] == info["last_units"] == info["last_tiles"] == 257
    assert info["last_split_chunks"] == 1
    check_log(plan, "dynamic", 257, K=K)
    assert_close_rows(p, c, [0, 5, M // 2, M - 1])
    plan.destroy()


def test_split_result_close_to_whole_tiles():
    # the split tile rounds differently (chunk partials summed in fp32), within tolerance
    M, N, K = 257 * 256, 256, 2048
    p = make_problem(M, N, K, "normal", seed=21)
    a = make_plan(256)
    b = make_plan(256, tail_split=4)
    say("case split vs whole")
    ca = run(p, a, "dynamic")
    cb = run(p, b, "dynamic")
    assert ptg.gemm_plan_info_get(b)["last_split_chunks"] == 4
    rows = list(range(256 * 256, M))
    assert_close_rows(p, cb, rows)
    assert np.array_equal(ca[: 256 * 256], cb[: 256 * 256])  # whole tiles: identical code and k order
    a.destroy()
    b.destroy()


@pytest.mark.parametrize("tile,q,policy", [(256, 0, 1), (256, 2, 0), (256, 1, 2), (128, 1, 1), (128, 2, 1)])
def test_tail_split_with_claim_options(tile, q, policy):
    # the split tail under other claim settings and the 128 tile: T = workers + 3 tiles
    torch = __import__("torch")
    plan = make_plan(tile, tail_split=4, claims_ahead=q, claim_policy=policy, log_capacity=4096)
    info = ptg.gemm_plan_info_get(plan)
    workers = info["occupancy"] * info["cu_count"]
    T = workers + 3
    M, N, K = T * tile, tile, 512 + 40
    p = make_problem(M, N, K, "uniform", seed=tile + q)
    say(f"case tail split tile={tile} claims_ahead={q} policy={policy} T={T}")
    c = run(p, plan, "dynamic")
    info = ptg.gemm_plan_info_get(plan)
    log = check_log(plan, "dynamic", info["last_items"], K=K, tiles=T)
    want = _expect_units(plan, log, T, workers, K, 4)
    rows = _split_rows(want, tile, M, 1) + [0, tile, M // 2]
    assert_close_rows(p, c, rows)
    plan.destroy()


@pytest.mark.parametrize("tile,shape", [(256, (2048, 2048, 8192)), (256, (700, 520, 1000)), (128, (1000, 776, 2056))])
def test_tail_split_underfilled_grid(tile, shape):
    """Fewer tiles than workers: the run is a single partial wave and every tile is split
    (K not a multiple of 32 in the ragged cases: the last chunk holds the partial k-step)."""
    M, N, K = shape
    p = make_problem(M, N, K, "normal" if K == 8192 else "uniform", seed=M + K)
    plan = make_plan(tile, tail_split=4, log_capacity=4096)
    info = ptg.gemm_plan_info_get(plan)
    workers = info["occupancy"] * info["cu_count"]
    tn = -(-N // tile)
    T = -(-M // tile) * tn
    assert T < workers
    rows = sorted(set(range(0, M, 7)) | {M - 1})
    outs = {}
    for mode in MODES:
        say(f"case tail split under-filled tile={tile} shape={shape} mode={mode}")
        c = run(p, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        S = info["last_split_chunks"]
        assert S >= 2 and info["last_tiles"] == T and info["last_items"] == T * S, info
        log = check_log(plan, mode, T * S, P=info["last_grid"] if mode == "static" else None, K=K, tiles=T)
        _expect_units(plan, log, T, workers, K, 4)
        assert_close_rows(p, c, rows)
        outs[mode] = c
    assert np.array_equal(outs["static"], outs["dynamic"])
    assert np.array_equal(outs["nonpersistent"], outs["dynamic"])
    plan.destroy()


@pytest.mark.parametrize("tile,shape", [(256, (2048, 2048, 8192)), (256, (2048, 2048, 2048)), (256, (257 * 256, 256, 4096)),
                                        (256, (512, 512, 16384)), (128, (300, 264, 16384)), (128, (1000, 776, 2056))])
def test_tail_split_auto(tile, shape):
    """tail_split = TAIL_SPLIT_AUTO: the run's chunk count is oracle.ownership.auto_split_chunks
    of its partial wave (1 = whole tiles), the units are split_units' with that count, and C
    matches the oracle; static and dynamic give the same bits."""
    from oracle.ownership import auto_split_chunks
    M, N, K = shape
    p = make_problem(M, N, K, "uniform", seed=M + K)
    plan = make_plan(tile, tail_split=ptg.TAIL_SPLIT_AUTO, log_capacity=4096)
    info = ptg.gemm_plan_info_get(plan)
    workers = info["occupancy"] * info["cu_count"]
    tn = -(-N // tile)
    T = -(-M // tile) * tn
    r = T % workers
    S = auto_split_chunks(r, -(-K // 32), info["cu_count"], tile)
    want_items = T - r + r * S if S > 1 else T
    outs = {}
    for mode in ("static", "dynamic"):
        say(f"case tail split auto tile={tile} shape={shape} mode={mode} (r={r}, S={S})")
        c = run(p, plan, mode)
        info = ptg.gemm_plan_info_get(plan)
        assert info["last_split_chunks"] == S and info["last_items"] == want_items, info
        log = check_log(plan, mode, want_items, P=info["last_grid"] if mode == "static" else None, K=K, tiles=T)
        want = _expect_units(plan, log, T, workers, K, S)
        rows = sorted(set(_split_rows(want, tile, M, tn)[::3]) | {0, M // 2, M - 1}) if S > 1 else [0, 1, M // 2, M - 1]
        assert_close_rows(p, c, rows)
        outs[mode] = c
    assert np.array_equal(outs["static"], outs["dynamic"])
    plan.destroy()

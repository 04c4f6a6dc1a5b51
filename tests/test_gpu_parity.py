"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Tolerance (the stated acceptance for bf16 inputs with fp32 accumulation):
relative Frobenius error <= 1e-3 and per element
|err| <= 1e-2 * sqrt(K) * max|a| * max|b| * 2^-8. Integer-valued inputs whose
partial sums stay below 2^24 are exact in fp32 and must match bit for bit;
identity and permutation operands must reproduce the other operand exactly.
The tile log must be exactly-once for every run (bit-exact ownership checks).
"""

import numpy as np
import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import (assert_close_full, check_log, make_plan, new_c, run, say, torch_mod, upload)
from workloads import f32_to_bf16_bits, make_problem
from oracle.gemm_ref import gemm_ref

pytestmark = pytest.mark.gpu

MODES = ("nonpersistent", "static", "dynamic")

# shapes spanning several tiles with ragged tails in M, N and K
SMALL_SHAPES = [
    (384, 512, 512),    # the twelve 128x128 tiles of the worked example
    (256, 256, 64),     # one 256 tile, two k-steps
    (1000, 776, 264),   # ragged M, N, K
    (513, 264, 72),
    (1, 8, 8),          # degenerate: one row, one k chunk
    (700, 1032, 1240),
]


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_shapes_all_modes(tile, shape):
    M, N, K = shape
    p = make_problem(M, N, K, "uniform", seed=M + N + K)
    plan = make_plan(tile)
    outs = {}
    for mode in MODES:
        say(f"case tile={tile} shape={shape} mode={mode}")
        c = run(p, plan, mode)
        assert_close_full(p, c)
        T = -(-M // tile) * -(-N // tile)
        info = ptg.gemm_plan_info_get(plan)
        check_log(plan, mode, T, P=info["last_grid"] if mode == "static" else None, K=K)
        outs[mode] = c
    # scheduling never changes numerics: same tile code, same k order
    assert np.array_equal(outs["static"], outs["dynamic"])
    assert np.array_equal(outs["nonpersistent"], outs["dynamic"])
    plan.destroy()


@pytest.mark.parametrize("tile", [128, 256])
def test_integer_inputs_bit_exact(tile):
    rng = np.random.default_rng(5)
    M, N, K = 520, 776, 1032  # |partial sums| <= 64 K < 2^24
    ai = rng.integers(-8, 9, size=(M, K))
    bi = rng.integers(-8, 9, size=(K, N))
    from workloads import GemmProblem
    p = GemmProblem(f32_to_bf16_bits(ai.astype(np.float32)), f32_to_bf16_bits(bi.astype(np.float32)))
    exact = (ai @ bi).astype(np.float32)
    plan = make_plan(tile)
    for mode in MODES:
        say(f"case integer tile={tile} mode={mode}")
        c = run(p, plan, mode)
        assert np.array_equal(c, exact)
    plan.destroy()


def test_identity_and_permutation_reproduce_operands():
    K = 512
    p = make_problem(K, 264, K, "normal", seed=9)
    eye = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    perm = np.random.default_rng(2).permutation(K)
    pm = f32_to_bf16_bits(np.eye(K, dtype=np.float32)[perm])
    from workloads import GemmProblem
    b_vals = ((p.b_bits.astype(np.uint32) << 16).view(np.float32))
    plan = make_plan(256)
    for mode in MODES:
        say(f"case identity mode={mode}")
        c = run(GemmProblem(eye, p.b_bits), plan, mode)
        assert np.array_equal(c, b_vals)
        c = run(GemmProblem(pm, p.b_bits), plan, mode)
        assert np.array_equal(c, b_vals[perm])
        # identity on the right reproduces A (rows of 264 are not a tile multiple)
        q = make_problem(300, K, K, "uniform", seed=4)
        c = run(GemmProblem(q.a_bits, eye), plan, mode)
        assert np.array_equal(c, (q.a_bits.astype(np.uint32) << 16).view(np.float32))
    plan.destroy()


def test_empty_and_degenerate_inputs():
    torch = torch_mod()
    plan = make_plan(256)
    A = torch.zeros((16, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
    # M == 0 / N == 0: nothing enqueued, C untouched
    C = new_c(0, 16)
    ptg.gemm_run(torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda"), B, C, plan)
    C2 = new_c(16, 0)
    ptg.gemm_run(A, torch.zeros((8, 0), dtype=torch.bfloat16, device="cuda"), C2, plan)
    # K == 0: C is all zeros
    for mode in MODES:
        C3 = new_c(300, 264)
        ptg.gemm_run(torch.zeros((300, 0), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((0, 264), dtype=torch.bfloat16, device="cuda"), C3, plan, mode=mode)
        torch.cuda.synchronize()
        assert torch.count_nonzero(C3).item() == 0 and not torch.isnan(C3).any().item()
    # shape errors come back as status codes, nothing is enqueued
    C4 = new_c(16, 12)
    st = ptg.gemm_run_raw(A.data_ptr(), torch.zeros((8, 12), dtype=torch.bfloat16, device="cuda").data_ptr(),
                          C4.data_ptr(), 16, 12, 8, plan)
    assert st == -2  # N not a multiple of 8
    assert ptg.gemm_run_raw(A.data_ptr(), B.data_ptr(), C4.data_ptr(), 16, 16, 12, plan) == -2  # K % 8
    assert ptg.gemm_run_raw(0, B.data_ptr(), C4.data_ptr(), 16, 16, 8, plan) == -1
    assert ptg.gemm_run_raw(A.data_ptr(), B.data_ptr(), C4.data_ptr(), 16, 16, 8, plan, mode=7) == -1
    assert ptg.gemm_run_raw(A.data_ptr() + 2, B.data_ptr(), C4.data_ptr(), 16, 16, 8, plan) == -1  # misaligned
    assert ptg.gemm_run_raw(A.data_ptr(), B.data_ptr(), C4.data_ptr(), -1, 16, 8, plan) == -2
    assert ptg.gemm_run_raw(A.data_ptr(), B.data_ptr(), C4.data_ptr(), 16, 16, (1 << 20) + 8, plan) == -2
    torch.cuda.synchronize()
    assert torch.isnan(C4).all().item()
    plan.destroy()


def test_plan_validation():
    for bad in ({"tile_edge": 256, "claims_ahead": 3}, {"tile_edge": 256, "ring_depth": 4},
                {"tile_edge": 256, "claim_policy": 3}, {"tile_edge": 256, "claim_lead": -1},
                {"tile_edge": 256, "ring_depth": 2, "claims_ahead": 2}, {"tile_edge": 256, "raster": 2},
                {"tile_edge": 256, "device": 99}):
        with pytest.raises(ptg.PtgError):
            ptg.gemm_create(**bad)
    d = ptg.gemm_default_desc(256, 0)
    d.bk = 64
    with pytest.raises(ptg.PtgError) as e:
        ptg.Plan(d)
    assert e.value.status == -3
    plan = ptg.gemm_create(tile_edge=256)
    info = ptg.gemm_plan_info_get(plan)
    assert info["cu_count"] > 0 and info["occupancy"] >= 1 and info["wallclock_khz"] > 0
    assert info["static_workers"] == info["occupancy"] * info["cu_count"]
    plan.destroy()


@pytest.mark.parametrize("policy", [0, 1, 2])
@pytest.mark.parametrize("q,depth", [(0, 3), (1, 3), (2, 3), (1, 2), (0, 2)])
def test_claims_ahead_variants(q, depth, policy):
    p = make_problem(1280, 1024, 512, "uniform", seed=q * 10 + depth)
    plan = make_plan(256, claims_ahead=q, ring_depth=depth, claim_policy=policy)
    say(f"case claims_ahead={q} depth={depth} policy={policy}")
    c = run(p, plan, "dynamic")
    assert_close_full(p, c)
    check_log(plan, "dynamic", 20)
    plan.destroy()


@pytest.mark.parametrize("group", [1, 3, 8])
def test_grouped_raster(group):
    p = make_problem(1800, 1288, 200, "uniform", seed=group)
    plan = make_plan(256, raster=1, raster_group=group)
    for mode in MODES:
        say(f"case raster group={group} mode={mode}")
        c = run(p, plan, mode)
        assert_close_full(p, c)
        T = 8 * 6
        info = ptg.gemm_plan_info_get(plan)
        check_log(plan, mode, T, P=info["last_grid"] if mode == "static" else None)
    plan.destroy()


def test_static_with_few_workers():
    # P smaller than the tile count: each worker walks w, w+P, ... (the tile sequence of the worked example)
    p = make_problem(1024, 1024, 256, "uniform", seed=3)
    plan = make_plan(256, static_workers=5)
    c = run(p, plan, "static")
    assert_close_full(p, c)
    log = check_log(plan, "static", 16, P=5)
    for w in range(5):
        assert sorted(log["tile"][log["worker"] == w].tolist()) == list(range(w, 16, 5))
    plan.destroy()


def test_logging_off_still_computes():
    p = make_problem(600, 520, 328, "uniform", seed=12)
    plan = ptg.gemm_create(tile_edge=128, log_capacity=0)
    for mode in MODES:
        c = run(p, plan, mode)
        assert_close_full(p, c)
    assert len(ptg.gemm_read_log(plan)) == 0
    plan.destroy()


def test_failure_forcing_counter_preset():
    # the counter starts at s: exactly tiles s..T-1 run, every worker's claims fail after that,
    # late slots exit at once, and the C rows of tiles < s are never written (stay NaN)
    torch = torch_mod()
    p = make_problem(2048, 512, 256, "uniform", seed=8)  # 8 x 2 tiles of 256
    T = 16
    plan = make_plan(256, claim_policy=0)
    for s in (0, 5, 15, 16, 40):
        say(f"case preset counter start={s}")
        A, B = upload(p)
        C = new_c(p.M, p.N)
        ptg.gemm_test_preset_counter(plan, s)
        ptg.gemm_run(A, B, C, plan, mode="dynamic")
        torch.cuda.synchronize()
        c = C.cpu().numpy()
        expected = list(range(s, T))
        check_log(plan, "dynamic", T, expected_tiles=expected)
        for k in range(T):
            mt, nt = divmod(k, 2)
            blk = c[mt * 256:(mt + 1) * 256, nt * 256:(nt + 1) * 256]
            if k >= s:
                assert not np.isnan(blk).any()
            else:
                assert np.isnan(blk).all()
    # the preset applies to one run only
    c = run(p, plan, "dynamic")
    assert_close_full(p, c)
    check_log(plan, "dynamic", T)
    plan.destroy()


@pytest.mark.parametrize("policy", [1, 2])
@pytest.mark.parametrize("shape,cap", [((1280, 1024, 128), 1), ((768, 768, 64), 2), ((256, 512, 64), 1)])
def test_xcd_regions_drained_by_stealing(shape, cap, policy):
    # with at most `cap` workers alive, the few workers must drain every XCD region
    # (interleaved or contiguous), most of them by stealing; T = 20, 9 and 2 leave
    # some regions empty or uneven
    M, N, K = shape
    p = make_problem(M, N, K, "uniform", seed=M + cap)
    plan = make_plan(256, claim_policy=policy, max_concurrent=cap, min_lds_bytes=96 * 1024)
    T = -(-M // 256) * -(-N // 256)
    say(f"case xcd stealing shape={shape} cap={cap} T={T} policy={policy}")
    c = run(p, plan, "dynamic")
    assert_close_full(p, c)
    log = check_log(plan, "dynamic", T)
    assert len(np.unique(log["worker"])) <= T
    plan.destroy()


@pytest.mark.parametrize("K", [32, 96, 320, 1000])
@pytest.mark.parametrize("q", [1, 2])
def test_claim_point_anywhere_in_the_tile(K, q):
    # The dynamic 256 x 256 main loop runs in two parts and sends its claims at the two-step trip
    # boundary at or before k-step nk - claim_lead: leads of 0 (last pair), 1, 2, 3 and past the
    # tile start, odd and even k-step counts (nk = 1, 3, 10, 32 with a K tail), one or two claims
    # ahead. Three workers at most, so each takes many tiles and every claim point recurs. The
    # result must equal the static run's bit for bit, and the log must be exactly-once.
    p = make_problem(1280, 1024, K, "uniform", seed=K + q)  # 5 x 4 tiles of 256
    T = 20
    plain = make_plan(256)
    say(f"case claim point K={K} claims_ahead={q}: static reference")
    ref = run(p, plain, "static")
    assert_close_full(p, ref)
    plain.destroy()
    for lead in (0, 1, 2, 3, 1000):
        for policy in (0, 1):
            plan = make_plan(256, claims_ahead=q, claim_lead=lead, claim_policy=policy, max_concurrent=3,
                             min_lds_bytes=96 * 1024)
            say(f"case claim point K={K} claims_ahead={q} lead={lead} policy={policy}")
            c = run(p, plan, "dynamic")
            assert np.array_equal(c, ref)
            log = check_log(plan, "dynamic", T, K=K)
            assert len(np.unique(log["worker"])) <= T
            plan.destroy()


@pytest.mark.parametrize("K", [8, 40, 136, 200, 232, 264, 488, 1000, 1240])
def test_k_tail_on_every_trip_boundary(K):
    # The 256 x 256 main loop uses load offsets computed once per tile for trips whose loads read whole
    # 32-deep slices, and recomputes them with the K-tail test from the first trip whose loads reach
    # the partial k-step. These K put that trip at every position: all trips (K = 8, 40, 136), from
    # the second trip (200, 232), later (264, 488, 1000, 1240), with odd and even k-step counts.
    p = make_problem(520, 776, K, "uniform", seed=K)  # 3 x 4 tiles of 256, ragged in M and N
    plan = make_plan(256)
    outs = {}
    for mode in MODES:
        say(f"case k tail K={K} mode={mode}")
        c = run(p, plan, mode)
        assert_close_full(p, c)
        info = ptg.gemm_plan_info_get(plan)
        check_log(plan, mode, 12, P=info["last_grid"] if mode == "static" else None, K=K)
        outs[mode] = c
    assert np.array_equal(outs["static"], outs["dynamic"])
    assert np.array_equal(outs["nonpersistent"], outs["dynamic"])
    plan.destroy()


def test_python_gemm_entry():
    # ptg.gemm(A, B, C=None, mode, plan): allocates C when absent, writes a given C in place, checks operands
    torch = torch_mod()
    p = make_problem(520, 264, 1000, "uniform", seed=51)
    A, B = ptg.bf16_from_bits(p.a_bits), ptg.bf16_from_bits(p.b_bits)
    for mode in MODES:
        say(f"case ptg.gemm mode={mode}")
        c = ptg.gemm(A, B, mode=mode)
        assert_close_full(p, c.cpu().numpy())
    C = torch.full((p.M, p.N), float("nan"), dtype=torch.float32, device="cuda")
    plan = make_plan(256, log_capacity=0)
    assert ptg.gemm(A, B, C, plan=plan) is C
    ptg.gemm_sync(plan)
    assert_close_full(p, C.cpu().numpy())
    with pytest.raises(ValueError):
        ptg.gemm(A.float(), B)                  # wrong dtype
    with pytest.raises(ValueError):
        ptg.gemm(A, B[:, :200])                  # not contiguous
    plan.destroy()


def _bits(rng, shape, exp, signed=True):
    """bf16 bit patterns with biased exponent field `exp` (0: subnormal) and random 7-bit mantissas
    (never zero for subnormals) and, when `signed`, random signs."""
    man = rng.integers(1 if exp == 0 else 0, 128, size=shape)
    sign = rng.integers(0, 2, size=shape) << 15 if signed else 0
    return ((exp << 7) | man | sign).astype(np.uint16)


@pytest.mark.parametrize("tile", [128, 256])
def test_subnormal_and_nonfinite_inputs(tile):
    """bf16 subnormal operands take part at full value (no flush to zero), fp32-subnormal
    products keep the fp32 subnormal spacing, and Inf / NaN / overflow come out as the
    rounded fp64 result says: IEEE products and sums rounded to fp32."""
    from workloads import GemmProblem
    rng = np.random.default_rng(21)
    M, N, K = 300, 264, 200
    plan = make_plan(tile)
    big = 127 + 100  # 2^100: subnormal x big lands in the normal fp32 range
    cases = {
        "subnormal A": GemmProblem(_bits(rng, (M, K), 0), _bits(rng, (K, N), big)),
        "subnormal B": GemmProblem(_bits(rng, (M, K), big), _bits(rng, (K, N), 0)),
    }
    for mode in MODES:
        for name, p in cases.items():
            say(f"case {name} tile={tile} mode={mode}")
            assert_close_full(p, run(p, plan, mode))
        # products near 2^-140: below the fp32 normal range; each rounding is to the subnormal spacing 2^-149
        say(f"case fp32-subnormal products tile={tile} mode={mode}")
        p = GemmProblem(_bits(rng, (M, K), 127 - 70), _bits(rng, (K, N), 127 - 70))
        c = run(p, plan, mode).astype(np.float64)
        ref = gemm_ref(p.a_bits, p.b_bits)
        assert np.abs(c - ref).max() <= K * 2.0 ** -149
        assert np.linalg.norm(c - ref) <= 1e-3 * np.linalg.norm(ref)
        # Inf, -Inf and NaN in A; a zero in B meets A's +Inf (Inf x 0 = NaN)
        say(f"case non-finite tile={tile} mode={mode}")
        a = _bits(rng, (M, K), 127, signed=False)
        b = _bits(rng, (K, N), 127)
        a[3, 17], a[290, 199], a[20, 5] = 0x7F80, 0xFF80, 0x7FC0
        b[17, 11] = 0x0000
        p = GemmProblem(a, b)
        c = run(p, plan, mode).astype(np.float64)
        with np.errstate(invalid="ignore"):
            ref = gemm_ref(a, b)
        for pred in (np.isnan, np.isposinf, np.isneginf):
            assert np.array_equal(pred(c), pred(ref)), pred.__name__
        assert np.isnan(c[20]).all() and np.isnan(c[3, 11]) and np.isinf(c[290]).all()
        fin = np.isfinite(ref)
        bound = 1e-2 * np.sqrt(K) * 2.0 * 2.0 * 2.0 ** -8
        assert np.abs(c[fin] - ref[fin]).max() <= bound
        # |exact| above the fp32 range rounds to Inf
        say(f"case overflow tile={tile} mode={mode}")
        p = GemmProblem(_bits(rng, (M, K), 127 + 70, signed=False), _bits(rng, (K, N), 127 + 70, signed=False))
        c = run(p, plan, mode)
        assert np.isposinf(c).all()
    plan.destroy()

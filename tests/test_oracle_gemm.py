"""Pins for the GEMM result oracle (CPU only).

The oracle is pinned to things other than itself: the bf16 format's definition
(known bit patterns), a library conversion routine (torch's bf16 -> float64 on
every bit pattern), brute force with correctly rounded sums on tiny shapes, exact
integer arithmetic, and closed forms (all-ones, identity, permutation). The
acceptance test is pinned by planting plausible mistakes (a dropped k term, a
transposed operand, a flipped sign, a shifted tile) that it must reject, and an
fp32-accumulated product that it must accept.
"""

import math

import numpy as np
import pytest
import torch

from oracle import gemm_ref as G
from workloads import f32_to_bf16_bits, make_problem


# (bits, value) from the bf16 layout: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits
KNOWN = [
    (0x0000, 0.0),
    (0x8000, -0.0),
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0x4000, 2.0),
    (0xC000, -2.0),
    (0x3F00, 0.5),
    (0x3FC0, 1.5),
    (0x4049, 3.140625),            # 1.1001001b * 2
    (0x0080, 2.0 ** -126),          # smallest normal
    (0x0001, 2.0 ** -133),          # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),    # largest subnormal
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


@pytest.mark.parametrize("bits,value", KNOWN)
def test_decode_known_patterns(bits, value):
    got = G.decode_bf16(np.array([bits], dtype=np.uint16))[0]
    assert got == value
    assert math.copysign(1.0, got) == math.copysign(1.0, value)


def test_decode_every_pattern_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = G.decode_bf16(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], t[~nan])
    # signed zeros agree too
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(t[~nan]))


@pytest.mark.parametrize("M,N,K,dist", [(1, 1, 1, "uniform"), (3, 5, 7, "uniform"), (4, 4, 64, "normal"),
                                        (8, 6, 513, "uniform"), (2, 3, 4096, "normal")])
def test_gemm_ref_matches_bruteforce(M, N, K, dist):
    p = make_problem(M, N, K, dist, seed=M * 1000 + K)
    ref = G.gemm_ref(p.a_bits, p.b_bits)
    bf = G.gemm_bruteforce(p.a_bits, p.b_bits)
    a = G.decode_bf16(p.a_bits)
    b = G.decode_bf16(p.b_bits)
    # float64 summation error bound: K * 2^-53 * sum |a b|
    bound = K * 2.0 ** -53 * (np.abs(a) @ np.abs(b))
    assert np.all(np.abs(ref - bf) <= bound + 1e-300)


def test_gemm_ref_integer_inputs_exact():
    rng = np.random.default_rng(7)
    M, N, K = 5, 6, 40
    ai = rng.integers(-8, 9, size=(M, K))
    bi = rng.integers(-8, 9, size=(K, N))
    a_bits = f32_to_bf16_bits(ai.astype(np.float32))
    b_bits = f32_to_bf16_bits(bi.astype(np.float32))
    ref = G.gemm_ref(a_bits, b_bits)
    exact = [[sum(int(ai[m, k]) * int(bi[k, n]) for k in range(K)) for n in range(N)] for m in range(M)]
    assert np.array_equal(ref, np.array(exact, dtype=np.float64))


def test_closed_forms():
    M, N, K = 7, 9, 33
    one = np.full((M, K), 0x3F80, dtype=np.uint16)
    oneb = np.full((K, N), 0x3F80, dtype=np.uint16)
    assert np.all(G.gemm_ref(one, oneb) == K)
    # identity A reproduces B; a permutation A permutes B's rows
    p = make_problem(K, N, K, "uniform", seed=3)
    eye = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    assert np.array_equal(G.gemm_ref(eye, p.b_bits), G.decode_bf16(p.b_bits))
    perm = np.random.default_rng(1).permutation(K)
    pm = f32_to_bf16_bits(np.eye(K, dtype=np.float32)[perm])
    assert np.array_equal(G.gemm_ref(pm, p.b_bits), G.decode_bf16(p.b_bits)[perm])
    # identity B reproduces A
    q = make_problem(M, K, K, "normal", seed=4)
    assert np.array_equal(G.gemm_ref(q.a_bits, eye), G.decode_bf16(q.a_bits))


def test_rows_and_elements_agree_with_bruteforce():
    p = make_problem(12, 10, 300, "uniform", seed=11)
    bf = G.gemm_bruteforce(p.a_bits, p.b_bits)
    rows = [0, 5, 11]
    r = G.gemm_ref_rows(p.a_bits, p.b_bits, rows)
    assert np.allclose(r, bf[rows], rtol=0, atol=1e-12)
    ri = np.array([0, 3, 11, 7])
    ci = np.array([9, 0, 4, 4])
    e = G.gemm_ref_elements(p.a_bits, p.b_bits, ri, ci)
    assert np.allclose(e, bf[ri, ci], rtol=0, atol=1e-12)


def _fp32_product(a_bits, b_bits):
    a = G.decode_bf16(a_bits).astype(np.float32)
    b = G.decode_bf16(b_bits).astype(np.float32)
    return (a @ b).astype(np.float64)


def test_acceptance_accepts_fp32_accumulation_and_rejects_planted_mistakes():
    M = N = K = 256
    p = make_problem(M, N, K, "uniform", seed=0)
    ref = G.gemm_ref(p.a_bits, p.b_bits)
    a = G.decode_bf16(p.a_bits)
    b = G.decode_bf16(p.b_bits)
    amax, bmax = float(np.abs(a).max()), float(np.abs(b).max())

    good = _fp32_product(p.a_bits, p.b_bits)
    assert G.check_result(good, ref, K, amax, bmax)["ok"]

    dropped = a[:, 1:] @ b[1:, :]                          # one k term missing
    assert not G.check_result(dropped, ref, K, amax, bmax)["ok"]
    transposed = a @ b.T                                   # B read transposed
    assert not G.check_result(transposed, ref, K, amax, bmax)["ok"]
    flipped = good.copy()
    flipped[17, 33] = -flipped[17, 33]                     # one sign wrong
    if abs(ref[17, 33]) > G.acceptance_bound(K, amax, bmax):
        assert not G.check_result(flipped, ref, K, amax, bmax)["ok"]
    shifted = np.roll(good, 128, axis=1)                   # tile written one tile over
    assert not G.check_result(shifted, ref, K, amax, bmax)["ok"]
    offk = a[:, list(range(1, K)) + [0]] @ b               # A's k index off by one
    assert not G.check_result(offk, ref, K, amax, bmax)["ok"]
    nan = good.copy()
    nan[0, 0] = np.nan
    assert not G.check_result(nan, ref, K, amax, bmax)["ok"]


def test_acceptance_bound_values():
    # worked-example shape: K = 512, U[-1,1] -> about 8.8e-4
    assert abs(G.acceptance_bound(512, 1.0, 1.0) - 1e-2 * math.sqrt(512) / 256) < 1e-15
    assert G.check_result(np.zeros((0, 3)), np.zeros((0, 3)), 8, 1.0, 1.0)["ok"]
    assert G.check_result(np.zeros((2, 2)), np.zeros((2, 2)), 0, 0.0, 0.0)["ok"]
    assert not G.check_result(np.ones((2, 2)), np.zeros((2, 2)), 4, 1.0, 1.0)["ok"]

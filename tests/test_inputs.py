"""The seeded input generator: bf16 rounding and determinism (CPU only)."""

import numpy as np
import torch

from workloads import f32_to_bf16_bits, grouped_k_values, make_problem, make_workload


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        rng.uniform(-1, 1, 200000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, -1e-45, np.inf, -np.inf], dtype=np.float32),
        # exact ties: low half == 0x8000, with even and odd kept bit
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00018000], dtype=np.uint32).view(np.float32),
    ])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_is_deterministic_and_shaped():
    p1 = make_problem(33, 17, 40, "normal", seed=5)
    p2 = make_problem(33, 17, 40, "normal", seed=5)
    assert p1.a_bits.shape == (33, 40) and p1.b_bits.shape == (40, 17)
    assert np.array_equal(p1.a_bits, p2.a_bits) and np.array_equal(p1.b_bits, p2.b_bits)
    p3 = make_problem(33, 17, 40, "normal", seed=6)
    assert not np.array_equal(p1.a_bits, p3.a_bits)


def test_distributions():
    p = make_problem(256, 256, 1024, "normal", seed=0)
    a = (p.a_bits.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(a.std()) * np.sqrt(1024) - 1.0) < 0.02
    u = make_problem(256, 256, 64, "uniform", seed=0)
    au = (u.a_bits.astype(np.uint32) << 16).view(np.float32)
    assert au.min() >= -1.0 and au.max() <= 1.0
    i = make_problem(16, 16, 16, "int", seed=0)
    ai = (i.a_bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(ai == np.round(ai)) and ai.min() >= -8 and ai.max() <= 8


def test_grouped_k_values_and_small_workloads():
    ks = grouped_k_values(0)
    assert len(ks) == 64 and ks.min() >= 512 and ks.max() <= 8192 and np.all(ks % 512 == 0)
    w = make_workload("worked_example")
    assert w.tile == 128 and w.problems[0].a_bits.shape == (384, 512) and w.problems[0].b_bits.shape == (512, 512)
    g = make_workload("grouped_uneven", groups=4)
    assert [p.K for p in g.problems] == grouped_k_values(0, groups=4).tolist()


def test_bf16_rounding_every_high_half_and_rounding_class():
    # the result depends only on the high 16 bits and on where the low 16 bits sit
    # against the halfway point 0x8000 (below, at, above); every high half is paired
    # with the low halves at and around those boundaries (NaN patterns excluded)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)

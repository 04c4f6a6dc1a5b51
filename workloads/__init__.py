"""Seeded synthetic inputs for the persistent tiled GEMM workloads.

This module only draws random numbers and rounds them to bf16 once; it holds none
of the GEMM or scheduling arithmetic. Both the CPU oracle and the HIP path receive
exactly the bit patterns produced here, so neither side re-rounds anything.

Workloads (shapes and distributions of the five measured configurations):

* ``worked_example``   M=384, N=512, K=512, A,B ~ U[-1,1], 128x128 tiles -> 12 tiles,
                       the twelve-tile, four-worker, three-slot example of the CLC blog
                       post (section on why a fixed task sequence tails).
* ``square_8192``      M=N=K=8192, A,B ~ N(0,1)/sqrt(K), 256x256 tiles -> 1024 tiles.
* ``tail_255/256/257`` N=256, K=4096, M = 255/256/257 * 256, A,B ~ U[-1,1].
* ``partial_occupancy`` the 8192^3 inputs, co-run with a spoiler (scheduling only).
* ``grouped_uneven``   64 problems, M=N=1024, K_g = 512 * U{1..16}, A_g,B_g ~ N(0,1)/sqrt(K_g).

Draw order (NumPy PCG64 ``default_rng(seed)``): A then B; for the grouped workload
the 64 K_g values first, then A_g, B_g per problem. Normals are drawn in float64,
scaled, cast to float32, then rounded to bf16 with round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "GemmProblem",
    "make_problem",
    "make_workload",
    "WORKLOADS",
    "grouped_k_values",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    NaN inputs map to a quiet NaN. Inputs here are finite by construction.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


@dataclasses.dataclass
class GemmProblem:
    """One GEMM C[M,N] = A[M,K] @ B[K,N] given as bf16 bit patterns (uint16, row-major)."""

    a_bits: np.ndarray  # (M, K) uint16
    b_bits: np.ndarray  # (K, N) uint16

    @property
    def M(self) -> int:
        return int(self.a_bits.shape[0])

    @property
    def K(self) -> int:
        return int(self.a_bits.shape[1])

    @property
    def N(self) -> int:
        return int(self.b_bits.shape[1])


def _draw(rng: np.random.Generator, shape, dist: str, k_scale: int) -> np.ndarray:
    if dist == "uniform":
        v = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        v = rng.standard_normal(size=shape) * (1.0 / np.sqrt(float(k_scale)))
    elif dist == "int":
        # small integers in [-8, 8]: exactly representable in bf16
        v = rng.integers(-8, 9, size=shape).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return f32_to_bf16_bits(v.astype(np.float32))


def make_problem(M: int, N: int, K: int, dist: str = "uniform", seed: int = 0,
                 rng: np.random.Generator | None = None) -> GemmProblem:
    """Draw A (M x K) then B (K x N) from ``dist`` with ``default_rng(seed)``."""
    if rng is None:
        rng = np.random.default_rng(seed)
    a = _draw(rng, (M, K), dist, K)
    b = _draw(rng, (K, N), dist, K)
    return GemmProblem(a, b)


def grouped_k_values(seed: int = 0, groups: int = 64, rng: np.random.Generator | None = None) -> np.ndarray:
    """K_g = 512 * U{1..16}, drawn first from the grouped workload's generator."""
    if rng is None:
        rng = np.random.default_rng(seed)
    return rng.integers(1, 17, size=groups).astype(np.int64) * 512


@dataclasses.dataclass
class Workload:
    name: str
    problems: List[GemmProblem]
    tile: int  # square output tile edge (BM = BN)

    @property
    def flops(self) -> float:
        return float(sum(2.0 * p.M * p.N * p.K for p in self.problems))


WORKLOADS = (
    "worked_example",
    "square_8192",
    "tail_255",
    "tail_256",
    "tail_257",
    "partial_occupancy",
    "grouped_uneven",
)


def make_workload(name: str, seed: int = 0, groups: int = 64) -> Workload:
    """Build one named workload from its recipe (see the module docstring)."""
    if name == "worked_example":
        return Workload(name, [make_problem(384, 512, 512, "uniform", seed)], 128)
    if name in ("square_8192", "partial_occupancy"):
        return Workload(name, [make_problem(8192, 8192, 8192, "normal", seed)], 256)
    if name in ("tail_255", "tail_256", "tail_257"):
        m_tiles = int(name.split("_")[1])
        return Workload(name, [make_problem(m_tiles * 256, 256, 4096, "uniform", seed)], 256)
    if name == "grouped_uneven":
        rng = np.random.default_rng(seed)
        ks = grouped_k_values(rng=rng, groups=groups)
        probs = [make_problem(1024, 1024, int(k), "normal", rng=rng) for k in ks]
        return Workload(name, probs, 256)
    raise ValueError(f"unknown workload {name!r}")

"""GEMM result oracle: C = A.B on bf16 inputs, accumulated in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed. The scheduling method changes only which worker computes which
output tile and when; each tile is one whole output block over the full K
extent and is computed exactly once ([CLC], section "from one tile per block to
one worker computing continuously": the work unit is a complete output tile, no
split-K or Stream-K; section "cancelling the launch, receiving the work
coordinate": each unit of work has exactly one owner). So the value of C is the
plain matrix product, independent of the schedule:

    C[m][n] = sum_k A[m][k] * B[k][n]

Inputs are the exact bf16 bit patterns sent to the GPU. A product of two bf16
numbers has at most 16 significant bits and is exact in float64; a float64 sum
of K <= 2^20 such terms is accurate to far below the acceptance bound, so the
float64 result stands in for the exact one.

Acceptance (the stated tolerance for the bf16-in / fp32-accumulate kernel):
  (i)  ||C_gpu - C_ref||_F / ||C_ref||_F <= 1e-3, in float64;
  (ii) for every element |C_gpu - C_ref| <= 1e-2 * sqrt(K) * max|a| * max|b| * 2^-8,
       with max|a|, max|b| over the whole A and B of that problem.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

__all__ = [
    "decode_bf16",
    "gemm_ref",
    "gemm_ref_rows",
    "gemm_ref_elements",
    "gemm_bruteforce",
    "acceptance_bound",
    "check_result",
]

REL_FROB_TOL = 1e-3
ELEM_COEF = 1e-2
BF16_UNIT = 2.0 ** -8


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 number is the upper half of an IEEE binary32 number: sign, 8-bit
    exponent, 7-bit fraction. Placing the 16 bits in the high half of a 32-bit
    word and reading it as binary32 gives the value; widening to float64 is exact.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen to NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_ref(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """float64 C = A @ B for row-major A (M x K) and B (K x N) given as bf16 bits."""
    a = decode_bf16(a_bits)
    b = decode_bf16(b_bits)
    if a.shape[1] != b.shape[0]:
        raise ValueError(f"inner dimensions differ: {a.shape} @ {b.shape}")
    return a @ b


def gemm_ref_rows(a_bits: np.ndarray, b_bits: np.ndarray, rows: Iterable[int]) -> np.ndarray:
    """float64 rows ``rows`` of A @ B (for sampled checks of very large problems)."""
    rows = np.asarray(list(rows), dtype=np.int64)
    a = decode_bf16(a_bits[rows])
    b = decode_bf16(b_bits)
    return a @ b


def gemm_ref_elements(a_bits: np.ndarray, b_bits: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """float64 C[rows[i], cols[i]] for paired index arrays, each as one dot product."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    a = decode_bf16(a_bits[rows])            # (S, K)
    b = decode_bf16(b_bits[:, cols]).T       # (S, K)
    return np.einsum("sk,sk->s", a, b)


def gemm_bruteforce(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Triple loop with correctly rounded sums (math.fsum) of the exact products.

    For tiny shapes only; used to pin ``gemm_ref`` to the definition.
    """
    a = decode_bf16(a_bits)
    b = decode_bf16(b_bits)
    M, K = a.shape
    N = b.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            out[m, n] = math.fsum(float(a[m, k]) * float(b[k, n]) for k in range(K))
    return out


def acceptance_bound(K: int, amax: float, bmax: float) -> float:
    """Per-element bound 1e-2 * sqrt(K) * max|a| * max|b| * 2^-8."""
    return ELEM_COEF * math.sqrt(max(K, 1)) * amax * bmax * BF16_UNIT


def check_result(c_gpu: np.ndarray, c_ref: np.ndarray, K: int, amax: float, bmax: float,
                 rel_tol: float = REL_FROB_TOL) -> Dict[str, object]:
    """Apply the two acceptance tests; return a report with an ``ok`` flag.

    ``c_gpu`` and ``c_ref`` must cover the same elements (a full matrix or a sample).
    ``amax`` and ``bmax`` are the largest magnitudes over the whole A and B.
    When C_ref is exactly zero everywhere the relative test is replaced by
    requiring C_gpu == 0 (the relative error is undefined there).
    """
    g = np.asarray(c_gpu, dtype=np.float64)
    r = np.asarray(c_ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    report: Dict[str, object] = {"elements": int(r.size)}
    if r.size == 0:
        report.update(ok=True, rel_frob=0.0, max_abs_err=0.0, bound=0.0)
        return report
    finite = bool(np.isfinite(g).all())
    diff = g - r
    ref_norm = float(np.linalg.norm(r.ravel()))
    err_norm = float(np.linalg.norm(diff.ravel())) if finite else math.inf
    if ref_norm == 0.0:
        rel = 0.0 if err_norm == 0.0 else math.inf
    else:
        rel = err_norm / ref_norm
    bound = acceptance_bound(K, amax, bmax)
    max_abs = float(np.max(np.abs(diff))) if finite else math.inf
    worst: Optional[tuple] = None
    if finite and r.ndim >= 1:
        worst = tuple(int(i) for i in np.unravel_index(int(np.argmax(np.abs(diff))), diff.shape))
    ok = finite and rel <= rel_tol and max_abs <= bound
    report.update(ok=bool(ok), rel_frob=rel, max_abs_err=max_abs, bound=bound, finite=finite, worst_index=worst)
    return report

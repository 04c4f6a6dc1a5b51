"""Helpers shared by the GPU tests: upload seeded inputs, run through the C ABI,
compare with the oracle, check the tile log."""

from __future__ import annotations

import sys

import numpy as np

import persistent_tiled_gemm_amd as ptg
from oracle.gemm_ref import check_result, decode_bf16, gemm_ref, gemm_ref_rows
from oracle.ownership import check_k_cover, check_ownership


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def upload(problem):
    A = ptg.bf16_from_bits(problem.a_bits)
    B = ptg.bf16_from_bits(problem.b_bits)
    return A, B


def new_c(M, N, fill=float("nan")):
    torch = torch_mod()
    return torch.full((M, N), fill, dtype=torch.float32, device="cuda")


def make_plan(tile=256, **kw):
    kw.setdefault("log_capacity", 1 << 14)
    return ptg.gemm_create(tile_edge=tile, **kw)


def run(problem, plan, mode, C=None, stream=None):
    A, B = upload(problem)
    if C is None:
        C = new_c(problem.M, problem.N)
    ptg.gemm_run(A, B, C, plan, mode=mode, stream=stream)
    torch_mod().cuda.synchronize()
    return C.cpu().numpy()


def maxabs(bits):
    return float(np.abs(decode_bf16(bits)).max()) if bits.size else 0.0


def assert_close_full(problem, c_gpu):
    ref = gemm_ref(problem.a_bits, problem.b_bits)
    rep = check_result(c_gpu, ref, problem.K, maxabs(problem.a_bits), maxabs(problem.b_bits))
    assert rep["ok"], rep
    return rep


def assert_close_rows(problem, c_gpu, rows):
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    ref = gemm_ref_rows(problem.a_bits, problem.b_bits, rows)
    rep = check_result(c_gpu[rows], ref, problem.K, maxabs(problem.a_bits), maxabs(problem.b_bits))
    assert rep["ok"], rep
    return rep


def check_log(plan, mode, T, P=None, expected_tiles=None, K=None, tiles=None, group=1):
    """Check the last run's log: T work items (== tiles unless the tail was split),
    the per-mode ownership rules on work-unit ids (unit u covers items [u*group,
    u*group + group): claim groups), and, given K, that the items of each of the
    `tiles` output tiles (default T) cover [0, K) exactly once."""
    log = ptg.gemm_read_log(plan)
    assert len(log) == T, (len(log), T)
    assert np.array_equal(log["unit"], np.arange(T) // group)
    policy = int(getattr(plan.desc, "claim_policy", 0))
    regions = 8 if policy in (1, 2) else 1
    layout = "contiguous" if policy == 2 else "interleaved"
    if group == 1:
        ran = log[log["visits"] > 0]
        errs = check_ownership(mode, T, ran["unit"], ran["worker"], ran["r0"].astype(np.float64),
                               ran["r1"].astype(np.float64), log["visits"], P=P, expected_tiles=expected_tiles,
                               regions=regions, region_layout=layout)
        assert not errs, errs
    else:
        # every item once; a unit's items run on one worker, back to back, in item order
        assert np.all(log["visits"] == 1), log["visits"]
        U = -(-T // group)
        worker = np.zeros(U, dtype=np.int64)
        start = np.zeros(U)
        end = np.zeros(U)
        for u in range(U):
            it = log[u * group:(u + 1) * group]
            assert len(np.unique(it["worker"])) == 1, (u, it["worker"])
            assert np.all(it["r0"][1:] >= it["r1"][:-1]), u
            worker[u], start[u], end[u] = it["worker"][0], it["r0"][0], it["r1"][-1]
        errs = check_ownership(mode, U, np.arange(U), worker, start, end, np.ones(U, dtype=np.int64), P=P,
                               regions=regions, region_layout=layout)
        assert not errs, errs
    if K is not None:
        ran = log[log["visits"] > 0]
        errs = check_k_cover(ran["tile"], ran["k_begin"], ran["k_end"], T if tiles is None else tiles, K)
        assert not errs, errs
    return log


def sample_rows(M, tile, rng, per_tile_row=1):
    """Rows to compare with the oracle: per_tile_row random rows of every tile row, plus the first and last."""
    rows = []
    for t in range(-(-M // tile)):
        lo, hi = t * tile, min(M, (t + 1) * tile)
        rows += rng.integers(lo, hi, size=per_tile_row).tolist()
    rows += [0, M - 1]
    return np.array(sorted(set(rows)))


class GroupedReference:
    """Oracle rows for every problem of a grouped run, computed once and checked
    against any number of runs: every C_g is NaN-free as a whole, and its sampled
    rows (every tile row of every problem) meet the acceptance bound."""

    def __init__(self, problems, seed, tile=256, per_tile_row=1):
        rng = np.random.default_rng(seed)
        self.problems = problems
        self.rows = [sample_rows(q.M, tile, rng, per_tile_row) for q in problems]
        self.refs = [gemm_ref_rows(q.a_bits, q.b_bits, r) for q, r in zip(problems, self.rows)]
        self.amax = [maxabs(q.a_bits) for q in problems]
        self.bmax = [maxabs(q.b_bits) for q in problems]

    def check(self, Cs, what=""):
        """Cs: the run's C_g, as device tensors or host arrays, in problem order."""
        torch = torch_mod()
        assert len(Cs) == len(self.problems)
        for g, (q, C) in enumerate(zip(self.problems, Cs)):
            if isinstance(C, np.ndarray):
                assert not np.isnan(C).any(), (what, g)
                got = C[self.rows[g]]
            else:
                assert not torch.isnan(C).any().item(), (what, g)
                got = C[torch.as_tensor(self.rows[g], device=C.device)].cpu().numpy()
            rep = check_result(got, self.refs[g], q.K, self.amax[g], self.bmax[g])
            assert rep["ok"], (what, g, rep)

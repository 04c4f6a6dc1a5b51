"""Checks of a per-tile ownership log against the schedulers' ownership rules.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A log holds one record per tile id: the worker (launch slot index) that ran it,
its start/end timestamps, and a visit count incremented atomically each time
any worker finished that tile. The rules:

* Every mode: each unit of work has exactly one owner ([CLC], section
  "cancelling the launch, receiving the work coordinate": the same coordinate
  never appears in two successful responses, so work either runs in its own
  launch or is taken by exactly one running worker). So visits == 1 for every
  tile handed out, 0 for every other, and a worker's tiles never overlap in time
  (a running block is never taken over, same section).
* Non-persistent: owner(k) = k (one block per tile; [CLC], section "from one
  tile per block ...", three-mode table).
* Static: owner(k) = k mod P and each worker's tiles run in increasing order
  ([CLC], section "why a fixed task sequence tails": W_i = i, i+4, i+8 for P = 4).
* Dynamic: any exactly-once owner map is valid (the claim order decides it);
  because claims come from one monotone counter each worker's tiles are
  strictly increasing in both id and start time. When tile ids are handed out
  by several counters, one per region of ids, the ids a worker takes from any
  one region are strictly increasing. Regions are interleaved (region r holds
  the ids k with k mod `regions` == r) or contiguous (region r holds the r-th
  of `regions` consecutive runs of ids, the first T mod `regions` runs one
  id longer than the rest).

Timestamps are taken on the GPU's constant-rate clock; makespan = latest tile
end - earliest tile start over the tiles that ran.

Split tails. When the tiles of a partial last wave are split along K (the
remedy for whole-tile quantisation that [CLC]'s first section names and leaves
out), the unit of ownership becomes the work unit: a whole tile, or one K-chunk
of a split tile. The rules above then hold for unit ids, and in addition the K
ranges of each tile's units must partition [0, K) exactly (check_k_cover):
every product a[m][k] b[k][n] enters C once.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import numpy as np

__all__ = ["check_ownership", "check_k_cover", "split_units", "auto_split_chunks", "makespan", "per_worker", "region_of"]


def per_worker(worker: np.ndarray, tiles: np.ndarray) -> Dict[int, np.ndarray]:
    out: Dict[int, List[int]] = {}
    for w, k in zip(worker.tolist(), tiles.tolist()):
        out.setdefault(int(w), []).append(int(k))
    return {w: np.asarray(v, dtype=np.int64) for w, v in out.items()}


def makespan(start: np.ndarray, end: np.ndarray) -> float:
    if len(start) == 0:
        return 0.0
    return float(np.max(end) - np.min(start))


def region_of(tile: np.ndarray, T: int, regions: int, layout: str = "interleaved") -> np.ndarray:
    """Region of each id under the interleaved or the contiguous layout."""
    tile = np.asarray(tile, dtype=np.int64)
    if layout == "interleaved":
        return tile % regions
    if layout != "contiguous":
        raise ValueError(f"unknown region layout {layout}")
    sizes = [T // regions + (1 if r < T % regions else 0) for r in range(regions)]
    ends = np.cumsum(sizes)
    return np.searchsorted(ends, tile, side="right")


def check_ownership(mode: str, T: int, tile: np.ndarray, worker: np.ndarray, start: np.ndarray,
                    end: np.ndarray, visits: np.ndarray, P: Optional[int] = None,
                    expected_tiles: Optional[Iterable[int]] = None, regions: int = 1,
                    region_layout: str = "interleaved") -> List[str]:
    """Return a list of violations (empty when the log obeys every rule).

    ``tile``, ``worker``, ``start``, ``end`` are per-record arrays for the tiles that
    ran (records of tiles that never ran must be dropped by the caller, using
    ``visits == 0``); ``visits`` is the full per-tile visit array of length T.
    ``expected_tiles`` is the set of tile ids that must have run (default all).
    """
    errs: List[str] = []
    tile = np.asarray(tile, dtype=np.int64)
    worker = np.asarray(worker, dtype=np.int64)
    start = np.asarray(start, dtype=np.float64)
    end = np.asarray(end, dtype=np.float64)
    visits = np.asarray(visits, dtype=np.int64)
    if len(visits) != T:
        errs.append(f"visits has length {len(visits)}, expected {T}")
        return errs
    expected = np.zeros(T, dtype=np.int64)
    if expected_tiles is None:
        expected[:] = 1
    else:
        for k in expected_tiles:
            expected[int(k)] = 1
    bad = np.nonzero(visits != expected)[0]
    if len(bad):
        errs.append(f"visit counts differ from exactly-once at {len(bad)} tiles, first {bad[:8].tolist()} "
                    f"(visits {visits[bad[:8]].tolist()})")
    ran = sorted(tile.tolist())
    want = sorted(np.nonzero(expected)[0].tolist())
    if ran != want:
        errs.append(f"logged tile set differs from expected ({len(ran)} logged, {len(want)} expected)")
    if np.any(end < start):
        errs.append("a tile ends before it starts")
    groups: Dict[int, List[int]] = {}
    for i, w in enumerate(worker.tolist()):
        groups.setdefault(int(w), []).append(i)
    for w, idx in groups.items():
        idx = sorted(idx, key=lambda i: (start[i], tile[i]))
        ks = tile[idx]
        st = start[idx]
        en = end[idx]
        if len(idx) > 1 and np.any(st[1:] < en[:-1]):
            errs.append(f"worker {w} runs two tiles at once")
        if mode == "static" or (mode == "dynamic" and regions <= 1):
            if len(ks) > 1 and np.any(np.diff(ks) <= 0):
                errs.append(f"worker {w} tiles not increasing in start order: {ks[:8].tolist()}")
        elif mode == "dynamic":
            reg = region_of(ks, T, regions, region_layout)
            for r in range(regions):
                kr = ks[reg == r]
                if len(kr) > 1 and np.any(np.diff(kr) <= 0):
                    errs.append(f"worker {w} tiles of region {r} not increasing: {kr[:8].tolist()}")
    if mode == "nonpersistent":
        if np.any(worker != tile):
            errs.append("non-persistent owner(k) != k")
        for w, idx in groups.items():
            if len(idx) != 1:
                errs.append(f"non-persistent worker {w} ran {len(idx)} tiles")
    elif mode == "static":
        if P is None or P < 1:
            errs.append("static check needs P")
        elif np.any(worker != tile % P):
            errs.append("static owner(k) != k mod P")
    elif mode != "dynamic":
        errs.append(f"unknown mode {mode}")
    return errs


def check_k_cover(tile: np.ndarray, k_begin: np.ndarray, k_end: np.ndarray, T: int, K) -> List[str]:
    """Violations of "the units of each tile cover its K range exactly once".

    ``tile``, ``k_begin``, ``k_end`` are per-unit arrays (units that ran); ``K`` is
    the reduction length, one int for all tiles or an array of length T.
    """
    errs: List[str] = []
    tile = np.asarray(tile, dtype=np.int64)
    kb = np.asarray(k_begin, dtype=np.int64)
    ke = np.asarray(k_end, dtype=np.int64)
    Ks = np.broadcast_to(np.asarray(K, dtype=np.int64), (T,))
    if np.any(ke < kb):
        errs.append("a unit ends its K range before it starts")
    spans: Dict[int, List[tuple]] = {}
    for t, b, e in zip(tile.tolist(), kb.tolist(), ke.tolist()):
        if not 0 <= t < T:
            errs.append(f"unit for tile {t} outside 0..{T - 1}")
            continue
        spans.setdefault(int(t), []).append((int(b), int(e)))
    for t in range(T):
        iv = sorted(spans.get(t, []))
        if not iv:
            errs.append(f"tile {t} has no unit")
            continue
        pos = 0
        for b, e in iv:
            if b != pos:
                errs.append(f"tile {t}: K range {'gap' if b > pos else 'overlap'} at {min(b, pos)}")
                break
            pos = e
        else:
            if pos != int(Ks[t]):
                errs.append(f"tile {t}: K covered up to {pos}, not {int(Ks[t])}")
    return errs


def auto_split_chunks(r: int, nk: int, cus: int, tile_edge: int = 256) -> int:
    """Chunk count S of the automatic split for r split tiles of nk k-steps on cus
    compute units. A rule of this implementation (the pages only name splitting
    along K as the cure for quantisation): the largest power of two S <= 8 such
    that every chunk gets an idle CU (r S <= cus) and at least min_steps k-steps,
    min_steps = 64 when 32 or more tiles split at once and 16 when fewer, times 4
    for 128 x 128 tiles; 1 (no split) when no S >= 2 qualifies.
    """
    if r <= 0:
        return 1
    min_steps = (64 if r >= 32 else 16) * (4 if tile_edge == 128 else 1)
    best = 1
    for S in (2, 4, 8):
        if r * S <= cus and nk // S >= min_steps:
            best = S
    return best


def split_units(T: int, workers: int, nk: int, max_chunks: int, min_chunk_steps: int = 4,
                max_split_tiles: int = 1024):
    """The work units of one run as (tile, first k-step, end k-step) triples, unit-id order.

    Tiles that fill whole waves of ``workers`` stay whole; each of the
    r = T mod workers tiles of the partial last wave is cut into
    S = min(max_chunks, workers // r, nk // min_chunk_steps) K-chunks when S >= 2,
    chunk c covering k-steps [floor(c nk / S), floor((c+1) nk / S)). Units of the
    split tiles follow the whole ones, tile-major. With T < workers the run is a
    single partial wave, and all T tiles are split.
    """
    whole = [(t, 0, nk) for t in range(T)]
    if max_chunks < 2 or workers < 2 or T == 0:
        return whole
    r = T % workers
    if r == 0 or r > max_split_tiles:
        return whole
    S = min(max_chunks, workers // r, nk // min_chunk_steps)
    if S < 2:
        return whole
    base = T - r
    units = [(t, 0, nk) for t in range(base)]
    for q in range(r):
        for c in range(S):
            units.append((base + q, (c * nk) // S, ((c + 1) * nk) // S))
    return units

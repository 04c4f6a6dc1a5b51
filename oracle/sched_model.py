"""Discrete-event model of the three tile schedulers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The model follows the pages' account of who computes which tile and when:

* Non-persistent: the grid has one block per output tile; hardware runs blocks in
  batches as resources free up; each block computes its own tile and exits
  ([CLC], section "from one tile per block to one worker computing continuously",
  the three-mode table, first row).
* Static persistent: the grid is a preset worker count P; worker i walks the
  fixed sequence i, i+P, i+2P, ... ([CLC], same table, second row, and the
  twelve-tile example in section "why a fixed task sequence tails"; [TS],
  section "WorkQueue", static mode fills exactly one wave).
* Dynamic persistent: the grid has one launch slot per tile; a running worker
  takes the next unstarted unit of work, each unit has exactly one owner, a
  running block's work is never taken over, a failed request ends only that
  worker's loop and a late-launched slot exits at once ([CLC], sections
  "cancelling the launch, receiving the work coordinate" and "cluster
  granularity and exit after failure"). On this hardware the unit is handed out
  by one atomic counter, so the claim order is the counter order.

Model assumptions (the pages ignore launch and scheduling overhead in their
example; both are parameters here, default 0):

1. ``S`` execution slots; slot s becomes usable at ``avail[s]`` (default 0).
2. Workgroups are dispatched in index order, each onto the earliest-free slot
   (ties -> lowest slot id), and hold the slot until they exit.
3. A workgroup starts working ``launch_cost`` after dispatch. A claim is an atomic
   read-and-increment performed at the moment it is issued; its value is usable
   ``claim_cost`` later. At one instant, dispatches come first; then events are
   taken in order of how many claims their workgroup has made so far, then by
   workgroup index (so every first claim at an instant precedes any prefetch
   claim at it).
4. Dynamic, ``claims_ahead`` q = 0: claim, wait for the value, run the tile, claim
   again when it ends. q >= 1: the first claim is made at entry; when a tile
   starts, claims are issued until q claims are outstanding beyond the current
   tile (the throttle); the next tile starts when the current one has ended and
   its claim value is back. A claim value >= T is a failure: the worker stops
   claiming and exits after the tile in hand. A claim is never issued after a
   failed one has been observed.
5. A running tile is never preempted.

Outputs: per tile (worker, slot, start, end), per workgroup (slot, dispatch,
exit), the makespan = latest tile end - earliest tile start, and the kernel span
= latest exit - earliest dispatch.
"""

from __future__ import annotations

import dataclasses
import heapq
import math
from collections import deque
from typing import Dict, List, Optional, Sequence

__all__ = ["TileRun", "WorkerRun", "Schedule", "simulate", "lpt_claim_order", "MODES"]

MODES = ("nonpersistent", "static", "dynamic")


@dataclasses.dataclass
class TileRun:
    tile: int
    worker: int
    slot: int
    start: float
    end: float


@dataclasses.dataclass
class WorkerRun:
    worker: int
    slot: int
    dispatch: float
    exit: float
    tiles: List[int]
    claims: int = 0


@dataclasses.dataclass
class Schedule:
    mode: str
    tiles: List[TileRun]           # indexed by tile id
    workers: Dict[int, WorkerRun]  # by workgroup index
    makespan: float
    span: float

    def owner(self) -> List[int]:
        return [r.worker for r in self.tiles]


def _check_invariants(T: int, tiles: List[Optional[TileRun]], workers: Dict[int, WorkerRun]) -> None:
    # exactly once: every tile has one run
    missing = [k for k in range(T) if tiles[k] is None]
    if missing:
        raise AssertionError(f"tiles never run: {missing[:10]}")
    seen = [0] * T
    for w in workers.values():
        prev_end = -math.inf
        for k in w.tiles:
            seen[k] += 1
            run = tiles[k]
            if run.worker != w.worker:
                raise AssertionError(f"tile {k} owner mismatch")
            if run.start < prev_end - 1e-12:
                raise AssertionError(f"worker {w.worker} overlaps itself at tile {k}")
            prev_end = run.end
    dup = [k for k in range(T) if seen[k] != 1]
    if dup:
        raise AssertionError(f"tiles run != once: {dup[:10]}")


def simulate(costs: Sequence[float], mode: str, slots: Optional[int] = None,
             avail: Optional[Sequence[float]] = None, P: Optional[int] = None,
             launch_cost: float = 0.0, claim_cost: float = 0.0, claims_ahead: int = 0,
             counter_start: int = 0, tie_rank: Optional[Sequence[int]] = None) -> Schedule:
    """Run the model. ``costs[k]`` is the duration of tile k (tiles in raster order).

    Exactly one of ``slots`` (all usable at time 0) or ``avail`` (per-slot start
    times) gives the execution slots. ``P`` is the static worker count (default:
    the number of slots). ``counter_start`` presets the dynamic claim counter
    (tiles below it are treated as already taken and are not run).
    ``tie_rank`` (a permutation of the workgroup indices) replaces the workgroup
    index as the tie-break between workgroup events at one instant with equal
    claim counts (assumption 3): any order in which simultaneous claims reach the
    counter can be modelled, the GPU's atomics resolving them in an order the
    model does not know.
    """
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}")
    T = len(costs)
    if avail is None:
        if slots is None or slots < 1:
            raise ValueError("need slots >= 1 or avail")
        avail = [0.0] * slots
    S = len(avail)
    if claims_ahead < 0:
        raise ValueError("claims_ahead must be >= 0")
    if mode == "static":
        G = P if P is not None else S
        if G < 1:
            raise ValueError("P must be >= 1")
    else:
        G = T
    if mode == "dynamic" and not (0 <= counter_start):
        raise ValueError("counter_start must be >= 0")
    rank = list(range(G)) if tie_rank is None else [int(r) for r in tie_rank]
    if sorted(rank) != list(range(G)):
        raise ValueError("tie_rank must be a permutation of the workgroup indices")

    tiles: List[Optional[TileRun]] = [None] * T
    workers: Dict[int, WorkerRun] = {}

    # event heap: (time, phase, key, seq, kind, payload)
    # phase 0 = slot frees (dispatch), key = slot id; phase 1 = workgroup events,
    # key (claims made so far, workgroup index). Dispatch at an instant precedes
    # the claims made at that instant.
    heap: list = []
    seq = [0]

    def push(time, phase, key, kind, payload):
        seq[0] += 1
        heapq.heappush(heap, (time, phase, key, seq[0], kind, payload))

    for s, a in enumerate(avail):
        push(float(a), 0, (s,), "slot_free", s)

    next_wg = [0]
    counter = [counter_start]

    # per-workgroup dynamic state
    pending: Dict[int, deque] = {}     # claim values in issue order: [value, ready_time]
    failed: Dict[int, bool] = {}

    def wkey(w: int):
        return (workers[w].claims, rank[w])

    def finish(w: int, now: float) -> None:
        workers[w].exit = now
        push(now, 0, (workers[w].slot,), "slot_free", workers[w].slot)

    def run_tile(w: int, k: int, start: float) -> float:
        end = start + float(costs[k])
        if tiles[k] is not None:
            raise AssertionError(f"tile {k} run twice")
        tiles[k] = TileRun(k, w, workers[w].slot, start, end)
        workers[w].tiles.append(k)
        return end

    def issue_claim(w: int, now: float) -> None:
        v = counter[0]
        counter[0] += 1
        workers[w].claims += 1
        pending[w].append([v, now + claim_cost])

    while heap:
        now, phase, key, _, kind, payload = heapq.heappop(heap)
        if kind == "slot_free":
            s = payload
            if next_wg[0] < G:
                w = next_wg[0]
                next_wg[0] += 1
                workers[w] = WorkerRun(w, s, now, now, [])
                push(now + launch_cost, 1, (0, rank[w]), "enter", w)
            continue
        w = payload
        if kind == "enter":
            if mode == "nonpersistent":
                if w < T:
                    end = run_tile(w, w, now)
                    push(end, 1, wkey(w), "exit", w)
                else:
                    finish(w, now)
            elif mode == "static":
                t = now
                k = w
                while k < T:
                    t = run_tile(w, k, t)
                    k += G
                push(t, 1, wkey(w), "exit", w)
            else:
                pending[w] = deque()
                failed[w] = False
                issue_claim(w, now)
                push(now + claim_cost, 1, wkey(w), "claim_ready", w)
        elif kind == "exit":
            finish(w, now)
        elif kind == "claim_ready":
            # the oldest outstanding claim's value is usable now
            v, ready = pending[w][0]
            if ready > now + 1e-15:
                push(ready, 1, wkey(w), "claim_ready", w)
                continue
            pending[w].popleft()
            if v >= T:
                failed[w] = True
                pending[w].clear()  # later values are failures too (monotone counter)
                finish(w, now)
                continue
            start = now
            if claims_ahead >= 1:
                while not failed[w] and len(pending[w]) < claims_ahead:
                    issue_claim(w, start)
            end = run_tile(w, v, start)
            push(end, 1, wkey(w), "tile_end", w)
        elif kind == "tile_end":
            if claims_ahead == 0:
                issue_claim(w, now)
                push(now + claim_cost, 1, wkey(w), "claim_ready", w)
            else:
                if not pending[w]:
                    finish(w, now)
                    continue
                v, ready = pending[w][0]
                if v >= T:
                    # observed failure: stop; never claim again
                    failed[w] = True
                    pending[w].clear()
                    finish(w, max(now, ready))
                    continue
                push(max(now, ready), 1, wkey(w), "claim_ready", w)
        else:  # pragma: no cover
            raise AssertionError(kind)

    if next_wg[0] != G:
        raise AssertionError("not all workgroups were dispatched")
    if mode == "dynamic" and counter_start > 0:
        # tiles below the preset were never handed out
        for k in range(min(counter_start, T)):
            tiles[k] = TileRun(k, -1, -1, math.nan, math.nan)
        run_tiles = [t for t in tiles if t is not None and t.worker >= 0]
        for k in range(counter_start, T):
            if tiles[k] is None:
                raise AssertionError(f"tile {k} never run")
    else:
        _check_invariants(T, tiles, workers)
        run_tiles = tiles  # type: ignore[assignment]
    if run_tiles:
        makespan = max(t.end for t in run_tiles) - min(t.start for t in run_tiles)
    else:
        makespan = 0.0
    span = (max(w.exit for w in workers.values()) - min(w.dispatch for w in workers.values())) if workers else 0.0
    return Schedule(mode, tiles, workers, makespan, span)  # type: ignore[arg-type]


def lpt_claim_order(problem_costs: Sequence[float], tiles_per_problem: Sequence[int]) -> List[int]:
    """Tile ids (problems numbered as given, tiles of problem g consecutive) in
    longest-processing-time claim order: problems by non-increasing per-tile cost,
    equal costs in the given problem order, each problem's tiles in their own order.

    [SKILL] (section "E - executable steps", choosing the scheduling mode) sends
    work of uneven cost to the dynamic scheduler; the order in which that work
    is handed out is not on the pages. Giving the costliest work out first is
    the classic longest-processing-time list-scheduling rule (Graham 1969),
    whose makespan is at most (4/3 - 1/(3S)) of the optimum on S slots.
    """
    starts = [0]
    for n in tiles_per_problem:
        starts.append(starts[-1] + int(n))
    order = sorted(range(len(problem_costs)), key=lambda g: (-float(problem_costs[g]), g))
    out: List[int] = []
    for g in order:
        out.extend(range(starts[g], starts[g + 1]))
    return out

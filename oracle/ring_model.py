"""Exhaustive interleaving checker for the claim / prefetch-ring protocol.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The protocol being checked is the one a workgroup of the HIP kernel runs; its
shape follows the pages:

* One elected producer (lane 0 of wave 0) issues the claim for the next tile and
  publishes the answer into a small ring of response records in shared memory;
  every wave of the workgroup consumes the records ([CLC], section "following
  the CUTLASS source": one elected thread issues requests, the warps that need
  coordinates are consumers, the scheduler warp consumes too; the example
  pipeline has depth 3, and a throttle bounds how far ahead the scheduler
  claims).
* Consumers wait, read the record for the next tile, check its success flag
  before using the coordinate, and release the stage for reuse ([CLC], same
  section: wait, read, decode, release; [TS], section "WorkQueue": the
  try-wait / wait / work / release tail).
* A failed claim ends the loop, no claim is issued after a failure has been
  observed, and a failed record carries no coordinate ([CLC], section "cluster
  granularity and exit after failure"; [SKILL], section "E", step 7: success
  is decided by a predicate, not a numeric sentinel).

Program of one workgroup with ``W`` waves, ring depth ``D``, claims-ahead ``q``,
``nb`` main-loop barriers per tile, and a claim counter that succeeds for the
first ``n_valid`` ordinals:

    producer:  issue(0); [write(0) happens asynchronously]; barrier(entry)
    all waves: read(0)
    for tile s = 0 .. n_valid-1:
        producer, q >= 1: at tile start issue every ordinal up to s+q not yet issued
                          (only if every earlier claim has returned valid)
        all waves: nb barriers (the main loop)
        producer, q == 0: issue(s+1)
        all waves: barrier(end of tile s); read(s+1); exit if it is a failure

``write(o)`` stores the record of ordinal o into slot o % D. It becomes possible
as soon as ordinal o has been issued and must happen before the producer
arrives at the next barrier that ends a tile (or the entry barrier for the
first claim): the claim's answer is back once the main loop's memory waits have
passed, and the producer publishes it before that barrier. At a tile start the
producer claims further ordinals (up to s+q) only when every claim from earlier
tiles, all of which have returned by then, was valid. The checker explores
every interleaving of the waves' steps and of the asynchronous writes and
reports the first violation of:

  R1  a read of ordinal o finds the record of ordinal o in slot o % D
      (not an older one, and not a newer one that overwrote it);
  R2  no claim is issued after a failed claim has returned;
  R3  every wave reaches its exit (no deadlock at a barrier).
"""

from __future__ import annotations

import dataclasses
import sys
from typing import Dict, List, Optional, Tuple

__all__ = ["RingResult", "check_ring_protocol", "wave_program"]


@dataclasses.dataclass
class RingResult:
    ok: bool
    states: int
    violation: Optional[str] = None


def wave_program(w: int, n_valid: int, q: int, nb: int) -> List[tuple]:
    """The op list of wave ``w`` (wave 0 is the producer)."""
    prog: List[tuple] = []
    issued = 0  # next ordinal to issue
    if w == 0:
        prog.append(("issue", (0,), ("entry",)))
        issued = 1
    prog.append(("barrier", ("entry",)))
    prog.append(("read", 0))
    for s in range(n_valid):
        if w == 0 and q >= 1 and issued - 1 < n_valid:
            # every claim from earlier tiles has returned valid: top up to s+q
            # (the claims of one top-up are issued together, before any answer is looked at)
            batch = tuple(range(issued, s + q + 1))
            if batch:
                prog.append(("issue", batch, ("end", s)))
                issued = s + q + 1
        for b in range(nb):
            prog.append(("barrier", ("k", s, b)))
        if w == 0 and q == 0:
            prog.append(("issue", (s + 1,), ("end", s)))
            issued = s + 2
        prog.append(("barrier", ("end", s)))
        prog.append(("read", s + 1))
    prog.append(("exit",))
    return prog


def check_ring_protocol(W: int, D: int, q: int, n_valid: int, nb: int = 1,
                        max_states: int = 2_000_000) -> RingResult:
    """Explore all interleavings; return the first violation found, if any."""
    if W < 1 or D < 1 or q < 0 or n_valid < 0 or nb < 0:
        raise ValueError("bad parameters")
    progs = [wave_program(w, n_valid, q, nb) for w in range(W)]
    # deadline of each write: the barrier named in its issue op
    deadline = {}
    for op in progs[0]:
        if op[0] == "issue":
            for o in op[1]:
                deadline[o] = op[2]

    # state: (pcs tuple, ring tuple of ordinals (-1 = empty), pending writes frozenset,
    #         returned ordinals frozenset, barrier arrivals frozenset of wave ids)
    start = (tuple(0 for _ in range(W)), tuple(-1 for _ in range(D)), frozenset(), frozenset(), frozenset())
    seen = set()
    stack = [start]
    sys.setrecursionlimit(10000)
    states = 0
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        states += 1
        if states > max_states:
            return RingResult(False, states, "state limit exceeded")
        pcs, ring, pend, returned, arrived = st
        if all(progs[w][pcs[w]][0] == "exit" for w in range(W)):
            continue
        moves = []
        # asynchronous writes of returned claims
        for o in pend:
            ring2 = list(ring)
            ring2[o % D] = o
            moves.append((pcs, tuple(ring2), pend - {o}, returned | {o}, arrived))
        for w in range(W):
            op = progs[w][pcs[w]]
            kind = op[0]
            if kind == "exit":
                continue
            pcs2 = list(pcs)
            if kind == "issue":
                batch = op[1]
                # R2: no earlier claim has returned a failure
                for e in returned:
                    if e < min(batch) and e >= n_valid:
                        return RingResult(False, states, f"R2: issue{batch} after failed claim {e} returned")
                pcs2[w] += 1
                moves.append((tuple(pcs2), ring, pend | frozenset(batch), returned, arrived))
            elif kind == "read":
                o = op[1]
                if ring[o % D] != o:
                    got = ring[o % D]
                    what = "empty" if got < 0 else ("stale" if got < o else "overwritten")
                    return RingResult(False, states, f"R1: wave {w} read({o}) found slot {o % D} {what} (ordinal {got})")
                pcs2[w] += 1
                moves.append((tuple(pcs2), ring, pend, returned, arrived))
            elif kind == "barrier":
                if w in arrived:
                    continue  # waiting
                if w == 0:
                    # producer must have published every record due at this barrier
                    for o in pend:
                        if deadline[o] == op[1]:
                            break
                    else:
                        o = None
                    if o is not None:
                        continue  # must write first (write moves are available)
                arr2 = arrived | {w}
                if len(arr2) == W:
                    # all waves arrived: release everyone past this barrier
                    for v in range(W):
                        if progs[v][pcs[v]] != op:
                            return RingResult(False, states, f"R3: waves at different barriers {op} vs {progs[v][pcs[v]]}")
                        pcs2[v] += 1
                    moves.append((tuple(pcs2), ring, pend, returned, frozenset()))
                else:
                    moves.append((pcs, ring, pend, returned, arr2))
        if not moves:
            return RingResult(False, states, f"R3: deadlock at pcs={pcs}")
        for m in moves:
            if m not in seen:
                stack.append(m)
    return RingResult(True, states)

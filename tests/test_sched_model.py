"""Pins for the discrete-event scheduler model (CPU only).

Pinned to: the pages' hand-worked example (tests/golden/worked_example.json),
closed forms for equal-cost tiles, Graham's list-scheduling bound (Graham 1966:
greedy list scheduling on S identical machines has makespan at most
sum(c)/S + (1 - 1/S) max(c), hence at most (2 - 1/S) OPT), the brute-force
optimum on tiny inputs, and small cases worked by hand in the comments.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle.sched_model import simulate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_makespans():
    g = _golden()
    costs = [g["tile_cost_t"]] * g["tiles"]
    S = g["concurrent_slots"]
    st = simulate(costs, "static", slots=S, P=g["planned_static_workers"])
    dy = simulate(costs, "dynamic", slots=S)
    dy1 = simulate(costs, "dynamic", slots=S, claims_ahead=1)
    npst = simulate(costs, "nonpersistent", slots=S)
    assert st.makespan == g["makespan_t"]["static"]
    assert dy.makespan == g["makespan_t"]["dynamic"]
    assert dy1.makespan == g["makespan_t"]["dynamic"]
    assert npst.makespan == g["makespan_t"]["nonpersistent"]
    # static sequences W_i = {i, i+4, i+8}
    for w, seq in enumerate(g["static_sequences"]):
        assert st.workers[w].tiles == seq
    # the three resident static workers finish at 3t, the fourth starts then
    assert max(st.workers[w].exit for w in range(3)) == g["static_first_three_finish_t"]
    assert st.workers[3].dispatch == g["static_first_three_finish_t"]
    # dynamic: three workers x four tiles; the other nine slots run nothing
    counts = sorted(len(w.tiles) for w in dy.workers.values())
    assert counts == [0] * 9 + [g["dynamic_tiles_per_worker"]] * 3


@pytest.mark.parametrize("T,S", [(1, 1), (7, 3), (12, 3), (12, 4), (255, 256), (256, 256), (257, 256), (1024, 256), (1024, 192)])
def test_equal_cost_closed_forms(T, S):
    t = 2.5
    costs = [t] * T
    want = math.ceil(T / S) * t
    assert simulate(costs, "nonpersistent", slots=S).makespan == pytest.approx(want)
    assert simulate(costs, "dynamic", slots=S).makespan == pytest.approx(want)
    assert simulate(costs, "dynamic", slots=S, claims_ahead=1).makespan == pytest.approx(want)
    for P in {1, max(1, S // 2), min(S, T)}:
        assert simulate(costs, "static", slots=S, P=P).makespan == pytest.approx(math.ceil(T / P) * t)


def test_hand_worked_uneven_case():
    # costs [3,1,1,1], 2 slots:
    #  dynamic: W0 takes 0 (0..3); W1 takes 1 (0..1), 2 (1..2), 3 (2..3) -> 3
    #  static P=2: W0 = {0,2} -> 4, W1 = {1,3} -> 2 -> 4
    #  non-persistent: B0 0..3, B1 0..1, B2 on slot1 1..2, B3 on slot1 2..3 -> 3
    c = [3, 1, 1, 1]
    assert simulate(c, "dynamic", slots=2).makespan == 3
    assert simulate(c, "static", slots=2, P=2).makespan == 4
    np_ = simulate(c, "nonpersistent", slots=2)
    assert np_.makespan == 3
    assert [r.slot for r in np_.tiles] == [0, 1, 1, 1]


def _opt(costs, S):
    best = math.inf
    for assign in itertools.product(range(S), repeat=len(costs)):
        loads = [0.0] * S
        for k, s in enumerate(assign):
            loads[s] += costs[k]
        best = min(best, max(loads))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_graham_bound_and_bruteforce_optimum(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(2, 8))
    S = int(rng.integers(1, 4))
    costs = rng.integers(1, 10, size=T).astype(float).tolist()
    dy = simulate(costs, "dynamic", slots=S)
    opt = _opt(costs, S)
    assert dy.makespan >= opt - 1e-12
    assert dy.makespan <= sum(costs) / S + (1 - 1 / S) * max(costs) + 1e-12
    assert dy.makespan <= (2 - 1 / S) * opt + 1e-12
    # every mode runs every tile exactly once (checked inside simulate) and never beats OPT
    for mode in ("static", "nonpersistent"):
        s = simulate(costs, mode, slots=S)
        assert s.makespan >= opt - 1e-12


def test_partial_occupancy_prediction():
    # 1024 equal tiles, 192 slots free at 0 and 64 more at the spoiler's end tau.
    # With 4t < tau: static (P = 256) runs 192 workers x 4 tiles to 4t, then the 64
    # blocked workers run 4 tiles each -> 8t. Dynamic: ceil(1024/192) = 6 -> 6t.
    t = 1.0
    tau = 10.0
    avail = [0.0] * 192 + [tau] * 64
    costs = [t] * 1024
    st = simulate(costs, "static", avail=avail, P=256)
    dy = simulate(costs, "dynamic", avail=avail)
    np_ = simulate(costs, "nonpersistent", avail=avail)
    assert st.makespan == 8 * t
    assert dy.makespan == 6 * t
    assert np_.makespan == 6 * t
    # with a short spoiler (tau = 2t) the freed slots join the dynamic run
    avail2 = [0.0] * 192 + [2 * t] * 64
    assert simulate(costs, "dynamic", avail=avail2).makespan == pytest.approx(5 * t)
    assert simulate(costs, "static", avail=avail2, P=256).makespan == pytest.approx(6 * t)


def test_launch_cost_is_amortised_by_persistence():
    # 12 tiles of t, 3 slots, launch cost l: non-persistent pays l per batch,
    # the persistent workers pay it once.
    t, l = 1.0, 0.25
    costs = [t] * 12
    npst = simulate(costs, "nonpersistent", slots=3, launch_cost=l)
    dy = simulate(costs, "dynamic", slots=3, launch_cost=l)
    assert npst.makespan == pytest.approx(4 * t + 3 * l)
    assert dy.makespan == pytest.approx(4 * t)


def test_claim_prefetch_hides_claim_latency():
    # q = 0 waits kappa before every tile; q = 1 claims at tile start, so with
    # kappa <= t only the first claim is exposed.
    t, kappa = 1.0, 0.3
    costs = [t] * 12
    q0 = simulate(costs, "dynamic", slots=3, claim_cost=kappa, claims_ahead=0)
    q1 = simulate(costs, "dynamic", slots=3, claim_cost=kappa, claims_ahead=1)
    assert q0.makespan == pytest.approx(4 * t + 3 * kappa)
    assert q1.makespan == pytest.approx(4 * t)
    q2 = simulate(costs, "dynamic", slots=3, claim_cost=kappa, claims_ahead=2)
    assert q2.makespan == pytest.approx(4 * t)


def test_claims_ahead_commits_work_early():
    # Uneven costs [5,1,1,1,1,1,1,1] on 2 slots, worked by hand:
    #  q = 0: W0 runs 0 (0..5); W1 runs 1..5 (0..5); at 5 both claim: W0 gets 6, W1 gets 7 -> 6
    #  q = 1: W0 claims 2 when tile 0 starts; W1 runs 1,3,4,5,6,7 (0..6); W0 runs 2 at 5..6 -> 6
    #  q = 2: W0 also holds 3: W0 runs 0 (0..5), 2 (5..6), 3 (6..7); W1 runs 1,4,5,6,7 -> 7
    costs = [5, 1, 1, 1, 1, 1, 1, 1]
    q0 = simulate(costs, "dynamic", slots=2, claims_ahead=0)
    q1 = simulate(costs, "dynamic", slots=2, claims_ahead=1)
    q2 = simulate(costs, "dynamic", slots=2, claims_ahead=2)
    assert q0.makespan == 6 and q0.workers[0].tiles == [0, 6]
    assert q1.makespan == 6 and q1.workers[0].tiles == [0, 2]
    assert q2.makespan == 7 and q2.workers[0].tiles == [0, 2, 3]
    assert q2.workers[1].tiles == [1, 4, 5, 6, 7]


def test_counter_preset_runs_only_the_remaining_tiles():
    costs = [1.0] * 10
    s = simulate(costs, "dynamic", slots=3, counter_start=6)
    ran = sorted(k for w in s.workers.values() for k in w.tiles)
    assert ran == [6, 7, 8, 9]
    s2 = simulate(costs, "dynamic", slots=3, counter_start=10)
    assert all(not w.tiles for w in s2.workers.values())


def test_late_slots_exit_at_once():
    costs = [1.0] * 6
    s = simulate(costs, "dynamic", slots=2)
    for w in s.workers.values():
        if not w.tiles:
            assert w.exit == w.dispatch  # one failed claim, nothing else
            assert w.claims == 1


def test_lpt_claim_order_definition():
    from oracle.sched_model import lpt_claim_order
    # problems 0..3 with 2, 1, 3, 1 tiles and per-tile costs 5, 9, 5, 1
    order = lpt_claim_order([5, 9, 5, 1], [2, 1, 3, 1])
    assert order == [2, 0, 1, 3, 4, 5, 6]
    # a permutation of all tiles, costs non-increasing along it
    rng = np.random.default_rng(4)
    costs = rng.integers(1, 17, size=40).tolist()
    n = rng.integers(1, 5, size=40).tolist()
    order = lpt_claim_order(costs, n)
    assert sorted(order) == list(range(sum(n)))
    owner = np.repeat(np.arange(40), n)
    seq = [costs[owner[t]] for t in order]
    assert all(a >= b for a, b in zip(seq, seq[1:]))


def test_lpt_order_meets_grahams_bound_and_helps_uneven_costs():
    from oracle.sched_model import lpt_claim_order
    # brute force on tiny instances: greedy dynamic over the LPT order stays within 4/3 - 1/(3S) of optimum
    rng = np.random.default_rng(7)
    for _ in range(30):
        S = int(rng.integers(2, 4))
        c = rng.integers(1, 10, size=int(rng.integers(3, 8))).tolist()
        order = lpt_claim_order(c, [1] * len(c))
        got = simulate([c[t] for t in order], "dynamic", slots=S).makespan
        best = min(max(sum(c[j] for j in range(len(c)) if a[j] == s) for s in range(S))
                   for a in itertools.product(range(S), repeat=len(c)))
        assert got <= (4 / 3 - 1 / (3 * S)) * best + 1e-9
    # the classic bad case for as-given order: short jobs first, one long job last
    c = [1] * 8 + [8]
    assert simulate(c, "dynamic", slots=4).makespan == 10
    order = lpt_claim_order(c, [1] * 9)
    assert simulate([c[t] for t in order], "dynamic", slots=4).makespan == 8


@pytest.mark.parametrize("q", [0, 1])
def test_every_tie_order_keeps_exactly_once_and_the_equal_cost_makespan(q):
    # Simultaneous claims reach the counter in an order the model cannot know (the GPU's atomics decide
    # it). Over every order of the workgroups at each instant (all permutations, T <= 6), every tile
    # still runs exactly once (asserted inside the model), each worker's tiles still increase, and with
    # equal costs on S free slots the makespan is still ceil(T / S) * t.
    import itertools
    for T in range(1, 7):
        for S in (1, 2, 3):
            for perm in itertools.permutations(range(T)):
                sch = simulate([1.0] * T, "dynamic", slots=S, claims_ahead=q, tie_rank=perm)
                assert sch.makespan == pytest.approx(math.ceil(T / S)), (T, S, perm, sch.makespan)
                for w in sch.workers.values():
                    assert w.tiles == sorted(w.tiles)


def test_tie_rank_must_be_a_permutation():
    with pytest.raises(ValueError):
        simulate([1.0] * 3, "dynamic", slots=2, tie_rank=[0, 0, 1])

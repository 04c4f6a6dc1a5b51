"""The ownership-log checker accepts the model's schedules and rejects planted errors (CPU)."""

import numpy as np

from oracle.ownership import check_ownership, makespan
from oracle.sched_model import simulate


def _log(sched, T):
    tile = np.array([r.tile for r in sched.tiles])
    worker = np.array([r.worker for r in sched.tiles])
    start = np.array([r.start for r in sched.tiles])
    end = np.array([r.end for r in sched.tiles])
    visits = np.ones(T, dtype=np.int64)
    return tile, worker, start, end, visits


def test_accepts_model_schedules():
    rng = np.random.default_rng(0)
    costs = rng.uniform(1, 3, size=40).tolist()
    for mode, kw in (("nonpersistent", {}), ("static", {"P": 7}), ("dynamic", {"claims_ahead": 1})):
        s = simulate(costs, mode, slots=5, **kw)
        tile, worker, start, end, visits = _log(s, 40)
        assert check_ownership(mode, 40, tile, worker, start, end, visits, P=7) == []
        assert makespan(start, end) == s.makespan


def test_rejects_planted_errors():
    s = simulate([1.0] * 12, "static", slots=3, P=4)
    tile, worker, start, end, visits = _log(s, 12)
    # duplicate visit
    v2 = visits.copy(); v2[5] = 2
    assert check_ownership("static", 12, tile, worker, start, end, v2, P=4)
    # lost tile
    assert check_ownership("static", 12, tile[1:], worker[1:], start[1:], end[1:],
                           np.r_[0, visits[1:]], P=4)
    # wrong static owner
    w2 = worker.copy(); w2[0] = 1
    assert check_ownership("static", 12, tile, w2, start, end, visits, P=4)
    # overlapping intervals on one worker
    st2 = start.copy(); st2[4] = start[0]
    assert check_ownership("dynamic", 12, tile, worker, st2, end, visits)
    # non-persistent owner must equal tile
    assert check_ownership("nonpersistent", 12, tile, worker, start, end, visits)
    # dynamic worker running tiles out of order
    d = simulate([1.0] * 6, "dynamic", slots=1)
    t, w, st, en, vi = _log(d, 6)
    t2 = t.copy(); t2[[1, 2]] = t2[[2, 1]]
    assert check_ownership("dynamic", 6, t2, w, st, en, vi)


def test_region_rule_for_partitioned_claims():
    # a worker that drains its own region (ids = 0 mod 2) and then steals from
    # region 1 takes decreasing ids overall but increasing ids per region
    tile = np.array([0, 2, 4, 1, 3])
    worker = np.zeros(5, dtype=np.int64)
    start = np.arange(5, dtype=float)
    end = start + 1
    visits = np.ones(5, dtype=np.int64)
    assert check_ownership("dynamic", 5, tile, worker, start, end, visits)            # one counter: violation
    assert not check_ownership("dynamic", 5, tile, worker, start, end, visits, regions=2)
    bad = np.array([2, 0, 4, 1, 3])                                                    # region 0 out of order
    assert check_ownership("dynamic", 5, bad, worker, start, end, visits, regions=2)

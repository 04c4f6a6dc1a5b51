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


def test_region_rule_for_contiguous_regions():
    # T = 5 in two contiguous regions {0, 1, 2} and {3, 4}: a worker that drains
    # region 1 and then steals region 0 from its start is valid; the same order
    # breaks the interleaved rule ({0, 2, 4}: 4 before 0) and the one-counter rule
    from oracle.ownership import region_of
    assert region_of(np.arange(5), 5, 2, "contiguous").tolist() == [0, 0, 0, 1, 1]
    assert region_of(np.arange(10), 10, 4, "contiguous").tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 3, 3]
    assert region_of(np.arange(3), 3, 8, "contiguous").tolist() == [0, 1, 2]
    tile = np.array([3, 4, 0, 1, 2])
    worker = np.zeros(5, dtype=np.int64)
    start = np.arange(5, dtype=float)
    end = start + 1
    visits = np.ones(5, dtype=np.int64)
    assert not check_ownership("dynamic", 5, tile, worker, start, end, visits, regions=2,
                               region_layout="contiguous")
    assert check_ownership("dynamic", 5, tile, worker, start, end, visits, regions=2)
    assert check_ownership("dynamic", 5, tile, worker, start, end, visits)
    bad = np.array([4, 3, 0, 1, 2])                                                    # region 1 out of order
    assert check_ownership("dynamic", 5, bad, worker, start, end, visits, regions=2, region_layout="contiguous")


def test_k_cover_accepts_partitions_and_rejects_planted_errors():
    from oracle.ownership import check_k_cover
    # three whole tiles and tile 3 cut into chunks [0,128) [128,320) [320,512)
    tile = np.array([0, 1, 2, 3, 3, 3])
    kb = np.array([0, 0, 0, 0, 128, 320])
    ke = np.array([512, 512, 512, 128, 320, 512])
    assert check_k_cover(tile, kb, ke, 4, 512) == []
    # order of the records does not matter
    p = np.array([5, 0, 3, 1, 4, 2])
    assert check_k_cover(tile[p], kb[p], ke[p], 4, 512) == []
    # a gap, an overlap, a short cover, a missing tile, a duplicated chunk
    assert check_k_cover(tile, kb, np.array([512, 512, 512, 120, 320, 512]), 4, 512)
    assert check_k_cover(tile, np.array([0, 0, 0, 0, 100, 320]), ke, 4, 512)
    assert check_k_cover(tile, kb, np.array([512, 512, 512, 128, 320, 500]), 4, 512)
    assert check_k_cover(tile[:-3], kb[:-3], ke[:-3], 4, 512)
    assert check_k_cover(np.r_[tile, 3], np.r_[kb, 320], np.r_[ke, 512], 4, 512)
    # K == 0: each tile is one empty unit
    assert check_k_cover(np.arange(3), np.zeros(3), np.zeros(3), 3, 0) == []
    # per-tile K (grouped problems)
    assert check_k_cover(np.array([0, 1]), np.array([0, 0]), np.array([64, 128]), 2, np.array([64, 128])) == []
    assert check_k_cover(np.array([0, 1]), np.array([0, 0]), np.array([64, 64]), 2, np.array([64, 128]))


def test_split_units_decomposition():
    from oracle.ownership import check_k_cover, split_units
    # 257 tiles on 256 workers, 64 k-steps, up to 8 chunks: the odd tile becomes 8 units of 8 k-steps
    u = split_units(257, 256, 64, 8)
    assert len(u) == 256 + 8
    assert u[:256] == [(t, 0, 64) for t in range(256)]
    assert u[256:] == [(256, 8 * c, 8 * c + 8) for c in range(8)]
    # chunk count limited by idle workers (r = 100 -> 256 // 100 = 2) and by K (nk // 4)
    assert len(split_units(356, 256, 64, 8)) == 256 + 100 * 2
    assert len(split_units(257, 256, 12, 8)) == 256 + 3          # nk // 4 = 3
    assert split_units(257, 256, 7, 8) == [(t, 0, 7) for t in range(257)]   # one chunk only: no split
    # no partial wave, splitting off
    assert split_units(512, 256, 64, 8) == [(t, 0, 64) for t in range(512)]
    assert split_units(257, 256, 64, 0) == [(t, 0, 64) for t in range(257)]
    # fewer tiles than workers: the one wave is partial and every tile splits
    # (100 tiles: 256 // 100 = 2 chunks; 64 tiles: 4 chunks fill all 256 workers)
    u = split_units(100, 256, 64, 8)
    assert u == [(t, 32 * c, 32 * c + 32) for t in range(100) for c in range(2)]
    assert len(split_units(64, 256, 64, 8)) == 256
    assert split_units(1, 256, 64, 8) == [(0, 8 * c, 8 * c + 8) for c in range(8)]
    assert split_units(0, 256, 64, 8) == []
    # uneven division of the k-steps still covers [0, nk) exactly
    for T, P, nk, s in ((257, 256, 30, 7), (14, 5, 13, 3), (1030, 256, 100, 64)):
        u = split_units(T, P, nk, s)
        t = np.array([x[0] for x in u]); b = np.array([x[1] for x in u]); e = np.array([x[2] for x in u])
        assert check_k_cover(t, b, e, T, nk) == []
        assert all(x[2] - x[1] >= 4 for x in u if x[2] - x[1] != nk)


def test_auto_split_chunks_is_the_largest_qualifying_power_of_two():
    """The automatic chunk count against its definition, checked by an independent
    search over every S in 1..8 on a grid of (r, nk, cus, tile edge), and at the
    design points measured on the part (whole tiles against S = 2 / 4 / 8)."""
    from oracle.ownership import auto_split_chunks
    for tile in (128, 256):
        for cus in (8, 64, 256):
            for r in (1, 2, 3, 7, 31, 32, 33, 64, 100, 256):
                for nk in (1, 15, 16, 31, 32, 63, 64, 65, 127, 128, 255, 256, 512, 1024, 4096):
                    S = auto_split_chunks(r, nk, cus, tile)
                    need = (64 if r >= 32 else 16) * (4 if tile == 128 else 1)
                    ok = [s for s in range(1, 9) if s & (s - 1) == 0 and (s == 1 or (r * s <= cus and nk // s >= need))]
                    assert S == max(ok), (tile, cus, r, nk, S, ok)
    assert auto_split_chunks(0, 256, 256) == 1
    # measured on MI355X (256 x 256 tiles unless stated; the best of whole / 2 / 4 / 8 chunks)
    assert auto_split_chunks(64, 256, 256) == 4          # 2048 x 2048 x 8192: 140 -> 98 us
    assert auto_split_chunks(64, 128, 256) == 2          # 2048 x 2048 x 4096: 78 -> 64 us
    assert auto_split_chunks(64, 64, 256) == 1           # 2048 x 2048 x 2048: no split pays
    assert auto_split_chunks(4, 512, 256) == 8           # 512 x 512 x 16384: 255 -> 70 us
    assert auto_split_chunks(32, 256, 256) == 4          # 8448 x 8192 x 8192 (32 tail tiles): 838 -> 794 us
    assert auto_split_chunks(1, 128, 256) == 8           # the 257-tile tail boundary: 205 -> 168 us
    assert auto_split_chunks(256, 256, 256, 128) == 1    # 2048 x 2048 x 8192 in 128 x 128 tiles: splitting lost
    assert auto_split_chunks(64, 256, 256, 128) == 1     # 1024 x 1024 x 8192 in 128 x 128 tiles: 4 chunks lost

"""The tile-log -> Chrome-trace converter (host-side formatting, CPU only)."""

import json

import numpy as np

import persistent_tiled_gemm_amd as ptg
from persistent_tiled_gemm_amd.trace import chrome_trace_events, write_chrome_trace


def _log():
    rec = np.zeros(4, dtype=ptg.TILE_REC_DTYPE)
    # three tiles that ran on two CUs of two XCDs, one unit that never ran
    rec["tile"] = [0, 1, 2, 3]
    rec["unit"] = [0, 1, 2, 3]
    rec["visits"] = [1, 1, 1, 0]
    rec["worker"] = [0, 1, 0, 0xFFFFFFFF]
    rec["xcc_id"] = [0, 1, 0, 0]
    rec["hw_id"] = [(5 << 8) | 3, (7 << 8) | 1, (5 << 8) | 3, 0]
    rec["r0"] = [1000, 1010, 1300, 0]
    rec["r1"] = [1250, 1260, 1500, 0]
    rec["t0"] = [0, 0, 0, 0]
    rec["t1"] = [5000, 5100, 4000, 0]
    rec["k_begin"] = [0, 0, 256, 0]
    rec["k_end"] = [512, 512, 512, 512]
    return rec


def test_events_follow_the_log():
    ev = chrome_trace_events(_log(), wallclock_khz=100000.0)   # 100 MHz: 10 ns per tick
    tiles = [e for e in ev if e["ph"] == "X"]
    assert len(tiles) == 3                                      # the unit that never ran is skipped
    assert {e["pid"] for e in ev if e["ph"] == "M"} == {0, 1}   # one process per XCD
    t0 = tiles[0]
    assert t0["pid"] == 0 and t0["tid"] == 5 and t0["ts"] == 0.0
    assert abs(t0["dur"] - 2.5) < 1e-12                         # 250 ticks of 10 ns
    assert t0["args"]["cycles"] == 5000
    t1 = tiles[1]
    assert t1["pid"] == 1 and t1["tid"] == 7 and abs(t1["ts"] - 0.1) < 1e-12
    assert "k[256,512)" in tiles[2]["name"]                      # a K-chunk is labelled with its range


def test_written_file_is_a_chrome_trace(tmp_path):
    path = tmp_path / "t.json"
    n = write_chrome_trace(_log(), 100000.0, str(path), metadata={"workload": "x"})
    doc = json.loads(path.read_text())
    assert n == 3 and len([e for e in doc["traceEvents"] if e["ph"] == "X"]) == 3
    assert doc["otherData"] == {"workload": "x"}


def test_empty_log():
    rec = np.zeros(2, dtype=ptg.TILE_REC_DTYPE)
    assert chrome_trace_events(rec, 100000.0) == []

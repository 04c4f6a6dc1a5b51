"""Tile log -> Chrome trace (chrome://tracing, Perfetto) converter.

Each logged work item becomes one complete ("X") event on the timeline of the
compute unit that ran it: process = XCD (the XCC_ID register), thread = CU
within it (the CU, SH and SE fields of HW_ID, bits 8..15), start and duration
from the constant-rate s_memrealtime stamps (r0, r1) in microseconds from the
earliest start. The event's arguments keep the tile, the unit that covered it,
its K range, the launch slot (worker) and the shader cycles it took (s_memtime).
Units that never ran (visits == 0) are skipped. Host-side formatting only: no
device code and no computation of the GEMM.
"""

from __future__ import annotations

import json
from typing import Optional

import numpy as np


def chrome_trace_events(records: np.ndarray, wallclock_khz: float, label: str = "gemm") -> list:
    """Trace events for the records of one run (the structured array gemm_read_log returns)."""
    ran = records[records["visits"] > 0]
    if len(ran) == 0:
        return []
    if wallclock_khz <= 0:
        raise ValueError("wallclock_khz must be positive")
    us_per_tick = 1e3 / float(wallclock_khz)
    base = int(ran["r0"].min())
    events = []
    for xcc in np.unique(ran["xcc_id"]):
        events.append({"name": "process_name", "ph": "M", "pid": int(xcc), "args": {"name": f"XCD {int(xcc)}"}})
    for r in ran:
        cu = (int(r["hw_id"]) >> 8) & 0xFF
        whole = int(r["k_begin"]) == 0
        events.append({
            "name": f"{label} tile {int(r['tile'])}" + ("" if whole else f" k[{int(r['k_begin'])},{int(r['k_end'])})"),
            "ph": "X",
            "pid": int(r["xcc_id"]),
            "tid": cu,
            "ts": (int(r["r0"]) - base) * us_per_tick,
            "dur": max(int(r["r1"]) - int(r["r0"]), 0) * us_per_tick,
            "args": {"tile": int(r["tile"]), "unit": int(r["unit"]), "k_begin": int(r["k_begin"]),
                     "k_end": int(r["k_end"]), "worker": int(r["worker"]), "problem": int(r["problem"]),
                     "cycles": int(r["t1"]) - int(r["t0"])},
        })
    return events


def write_chrome_trace(records: np.ndarray, wallclock_khz: float, path: str, label: str = "gemm",
                       metadata: Optional[dict] = None) -> int:
    """Write the run's trace to `path` (JSON object format); return the number of tile events."""
    events = chrome_trace_events(records, wallclock_khz, label)
    doc = {"traceEvents": events, "displayTimeUnit": "ms"}
    if metadata:
        doc["otherData"] = metadata
    with open(path, "w") as f:
        json.dump(doc, f)
    return sum(1 for e in events if e["ph"] == "X")

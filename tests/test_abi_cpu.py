"""The C-ABI library loads and exports every function include/ptg_gemm.h declares (CPU only).

No compute call is made here; only argument checks that return before any HIP
call (null handles, bad enums, descriptor defaults) are exercised.
"""

import ctypes
import os
import re
import subprocess

import pytest

import persistent_tiled_gemm_amd as ptg

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ptg_gemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(gemm_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ptg.LIB_PATH):
        pytest.fail(f"{ptg.LIB_PATH} not built (run python -m persistent_tiled_gemm_amd.build)")
    return ptg.load_library()


def test_header_declares_the_abi():
    names = _declared_functions()
    assert set(names) == set(ptg.ABI_FUNCTIONS), names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ptg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(gemm_[a-z_0-9]+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings_and_defaults(lib):
    assert ptg.gemm_status_str(0) == "ok"
    for s in range(-8, 0):
        assert ptg.gemm_status_str(s) not in ("", "unknown status")
    assert ptg.gemm_status_str(-99) == "unknown status"
    d = ptg.gemm_default_desc(256, 0)
    assert (d.bm, d.bn, d.bk, d.ring_depth, d.claims_ahead, d.claim_lead, d.claim_policy) == (256, 256, 32, 3, 1, 4, 1)
    assert (d.log_capacity, d.max_concurrent, d.gate_spin_limit, d.tail_split, d.claim_group) == (0, 0, 0, 0, 1)
    assert (d.k_rotation, d.dynamic_grid) == (ptg.KROT_AUTO, ptg.GRID_ALL)   # one launch slot per tile
    d = ptg.gemm_default_desc(128, 0)
    assert (d.bm, d.bn) == (128, 128)
    with pytest.raises(ptg.PtgError):
        ptg.gemm_default_desc(192, 0)


def test_descriptor_values_out_of_range_are_rejected_before_any_hip_call(lib):
    for field, bad in (("dynamic_grid", 2), ("dynamic_grid", -1), ("k_rotation", 5), ("claim_policy", 3),
                       ("tail_split", -2), ("tail_split", 65)):
        d = ptg.gemm_default_desc(256, 0)
        setattr(d, field, bad)
        out = ctypes.c_void_p()
        assert lib.gemm_create(ctypes.byref(out), ctypes.byref(d)) == -1, field
        assert not out.value


def test_null_arguments_are_rejected_before_any_hip_call(lib):
    assert lib.gemm_create(None, None) == -1
    assert lib.gemm_run(None, None, None, 8, 8, 8, 2, None, None) == -1
    assert lib.gemm_run_noalloc(None, None, None, 8, 8, 8, 2, None, None) == -1
    assert lib.gemm_run_noalloc(None, None, None, 8, 8, 8, 7, None, None) == -1
    assert lib.gemm_run_grouped(1, None, None, None, None, None, None, 2, None, None) == -1
    n = ctypes.c_size_t(0)
    assert lib.gemm_read_log(None, None, 0, ctypes.byref(n)) == -1
    assert lib.gemm_plan_info_get(None, None) == -1
    assert lib.gemm_destroy(None) == 0
    assert lib.gemm_test_preset_counter(None, 3) == -1
    assert lib.gemm_test_preset_gate(None, 3) == -1
    assert lib.gemm_sync(None) == -1
    assert lib.gemm_test_stream_destroy(None) == -1
    assert lib.gemm_test_stream_cu_mask(None, 0, None, 0) == -1
    assert lib.gemm_last_hip_error(None) == b""
    assert lib.gemm_test_spoiler(0, 0, 1000, None, None, 0.0) == -1
    assert lib.gemm_mfma_probe(0, 100, 1, 16, None, None) == -1
    assert lib.gemm_hbm_probe(0, 1 << 30, 0, 20, None) == -1


def test_struct_layouts_match_the_binding(tmp_path):
    # compile the header as plain C and compare sizes and field offsets with ctypes
    structs = {"gemm_tile_desc": ptg.TileDesc, "gemm_tile_rec": ptg.TileRec, "gemm_plan_info": ptg.PlanInfo}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "ptg_gemm.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                               check=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[f"{cname} size"]) == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert int(got[f"{cname}.{field}"]) == getattr(cls, field).offset, (cname, field)
    assert ptg.TILE_REC_DTYPE.itemsize == ctypes.sizeof(ptg.TileRec)
    for field in ptg.TILE_REC_DTYPE.names:
        assert ptg.TILE_REC_DTYPE.fields[field][1] == getattr(ptg.TileRec, field).offset, field

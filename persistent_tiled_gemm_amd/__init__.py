"""Python binding of the persistent tiled bf16 GEMM C ABI (include/ptg_gemm.h).

Argument marshalling only: every step of the GEMM and of its tile schedulers
runs in the HIP library libptg_gemm.so built in this directory. There is no
fallback; if the library is missing, loading it raises.

The function names are the C ABI's: gemm_default_desc, gemm_create, gemm_run,
gemm_run_noalloc, gemm_run_grouped, gemm_read_log, gemm_sync, gemm_plan_info_get, gemm_destroy,
gemm_status_str, gemm_last_hip_error, gemm_test_preset_counter,
gemm_test_preset_gate, gemm_test_stream_cu_mask, gemm_test_stream_destroy,
gemm_test_spoiler, gemm_mfma_probe, gemm_hbm_probe. Tensors are torch device tensors: A and B
bf16 (or int16 / uint16 views of bf16 bits), C float32, all contiguous; streams
are torch.cuda streams (default: the current stream).
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libptg_gemm.so")

SCHED_NONPERSISTENT = 0
SCHED_STATIC = 1
SCHED_DYNAMIC = 2
MODES = {"nonpersistent": SCHED_NONPERSISTENT, "static": SCHED_STATIC, "dynamic": SCHED_DYNAMIC}

# K orders (plan field k_rotation)
KROT_AUTO, KROT_OFF, KROT_XCD, KROT_XCD2, KROT_UNIT = 0, 1, 2, 3, 4
GRID_ALL, GRID_RESIDENT = 0, 1  # gemm_tile_desc.dynamic_grid
TAIL_SPLIT_AUTO = -1  # gemm_tile_desc.tail_split: the library picks the chunk count per run

GEMM_OK = 0
STATUS_NAMES = {0: "GEMM_OK", -1: "GEMM_E_INVALID_ARG", -2: "GEMM_E_SHAPE", -3: "GEMM_E_UNSUPPORTED",
                -4: "GEMM_E_DEVICE", -5: "GEMM_E_HIP", -6: "GEMM_E_NOMEM", -7: "GEMM_E_TIMEOUT",
                -8: "GEMM_E_SCHED"}

# exported names, in the order of the header
ABI_FUNCTIONS = ("gemm_default_desc", "gemm_create", "gemm_run", "gemm_run_noalloc", "gemm_run_grouped", "gemm_read_log",
                 "gemm_sync", "gemm_plan_info_get", "gemm_destroy", "gemm_status_str", "gemm_last_hip_error",
                 "gemm_test_preset_counter", "gemm_test_preset_gate", "gemm_test_stream_cu_mask",
                 "gemm_test_stream_destroy", "gemm_test_spoiler", "gemm_mfma_probe", "gemm_hbm_probe")


class PtgError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        msg = f"{what}: {STATUS_NAMES.get(status, status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


class TileDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "bm", "bn", "bk", "ring_depth", "claims_ahead", "claim_lead", "claim_policy", "raster", "raster_group", "static_workers",
        "log_capacity", "min_lds_bytes", "max_concurrent", "max_groups", "device", "tail_split", "group_order", "claim_group",
        "b_layout", "gate_spin_limit", "k_rotation", "dynamic_grid")]


class TileRec(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_uint32), ("worker", ctypes.c_uint32), ("hw_id", ctypes.c_uint32),
                ("xcc_id", ctypes.c_uint32), ("t0", ctypes.c_uint64), ("t1", ctypes.c_uint64),
                ("r0", ctypes.c_uint64), ("r1", ctypes.c_uint64), ("visits", ctypes.c_uint32),
                ("problem", ctypes.c_uint32), ("unit", ctypes.c_uint32), ("k_begin", ctypes.c_uint32),
                ("k_end", ctypes.c_uint32), ("pad", ctypes.c_uint32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("cu_count", ctypes.c_int32), ("occupancy", ctypes.c_int32),
                ("static_workers", ctypes.c_int32), ("wallclock_khz", ctypes.c_int64),
                ("last_tiles", ctypes.c_int64), ("last_units", ctypes.c_int64), ("last_items", ctypes.c_int64), ("last_split_base", ctypes.c_int64),
                ("last_split_chunks", ctypes.c_int32), ("last_claim_group", ctypes.c_int32),
                ("last_grid", ctypes.c_int64), ("last_mode", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("last_k_rotation", ctypes.c_int32), ("pad", ctypes.c_int32)]


TILE_REC_DTYPE = np.dtype([("tile", "<u4"), ("worker", "<u4"), ("hw_id", "<u4"), ("xcc_id", "<u4"),
                           ("t0", "<u8"), ("t1", "<u8"), ("r0", "<u8"), ("r1", "<u8"),
                           ("visits", "<u4"), ("problem", "<u4"), ("unit", "<u4"), ("k_begin", "<u4"),
                           ("k_end", "<u4"), ("pad", "<u4")])
assert TILE_REC_DTYPE.itemsize == ctypes.sizeof(TileRec) == 72

_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libptg_gemm.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is missing: build it with `python -m persistent_tiled_gemm_amd.build`")
    # torch brings its own HIP runtime with the same soname as the system one the
    # library is linked against; whichever loads first serves the whole process.
    # Importing torch first makes that torch's, so the library and the caller's
    # tensors and streams share one runtime (the other order leaves torch unable
    # to see the GPU).
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the library is still usable from C
        pass
    lib = ctypes.CDLL(p)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    P64 = ctypes.POINTER(ctypes.c_int64)
    lib.gemm_default_desc.argtypes = [ctypes.POINTER(TileDesc), i32, i32]
    lib.gemm_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(TileDesc)]
    lib.gemm_run.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.gemm_run_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.gemm_run_grouped.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                     P64, P64, P64, i32, vp, vp]
    lib.gemm_read_log.argtypes = [vp, ctypes.POINTER(TileRec), ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.gemm_sync.argtypes = [vp]
    lib.gemm_plan_info_get.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_status_str.argtypes = [i32]
    lib.gemm_status_str.restype = ctypes.c_char_p
    lib.gemm_last_hip_error.argtypes = [vp]
    lib.gemm_last_hip_error.restype = ctypes.c_char_p
    lib.gemm_test_preset_counter.argtypes = [vp, u32]
    lib.gemm_test_preset_gate.argtypes = [vp, u32]
    lib.gemm_test_stream_cu_mask.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(u32), u32]
    lib.gemm_test_stream_destroy.argtypes = [vp]
    lib.gemm_test_spoiler.argtypes = [i32, i32, i64, vp, vp, ctypes.c_double]
    lib.gemm_mfma_probe.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]
    lib.gemm_hbm_probe.argtypes = [i32, i64, i32, i32, ctypes.POINTER(ctypes.c_double)]
    for name in ABI_FUNCTIONS:
        if name not in ("gemm_status_str", "gemm_last_hip_error"):
            getattr(lib, name).restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def _check(status: int, what: str, plan=None) -> None:
    if status != GEMM_OK:
        detail = ""
        lib = load_library()
        if plan is not None and plan._handle:
            detail = (lib.gemm_last_hip_error(plan._handle) or b"").decode()
        if not detail:
            detail = (lib.gemm_status_str(status) or b"").decode()
        raise PtgError(status, what, detail)


def gemm_status_str(status: int) -> str:
    return (load_library().gemm_status_str(int(status)) or b"").decode()


def gemm_default_desc(tile_edge: int = 256, device: int = 0) -> TileDesc:
    d = TileDesc()
    _check(load_library().gemm_default_desc(ctypes.byref(d), int(tile_edge), int(device)), "gemm_default_desc")
    return d


class Plan:
    """A gemm_tile_cfg handle (owns the library scratch)."""

    def __init__(self, desc: TileDesc):
        self._handle = ctypes.c_void_p()
        self.desc = desc
        _check(load_library().gemm_create(ctypes.byref(self._handle), ctypes.byref(desc)), "gemm_create")

    def destroy(self) -> None:
        if self._handle:
            load_library().gemm_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()

    @property
    def handle(self):
        return self._handle


def gemm_create(desc: Optional[TileDesc] = None, **fields) -> Plan:
    """gemm_create: build a plan from a descriptor (or defaults overridden by fields)."""
    if desc is None:
        desc = gemm_default_desc(fields.pop("tile_edge", 256), fields.get("device", 0))
    for k, v in fields.items():
        setattr(desc, k, int(v))
    return Plan(desc)


def gemm_destroy(plan: Plan) -> None:
    plan.destroy()


def gemm_last_hip_error(plan: Plan) -> str:
    return (load_library().gemm_last_hip_error(plan.handle) or b"").decode()


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_operands(A, B, C, b_layout: int = 0):
    import torch
    for name, t, dts in (("A", A, (torch.bfloat16, torch.int16, torch.uint16)),
                         ("B", B, (torch.bfloat16, torch.int16, torch.uint16)), ("C", C, (torch.float32,))):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype not in dts:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dts}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D")
    M, K = A.shape
    K2, N = B.shape if b_layout == 0 else tuple(B.shape)[::-1]  # b_layout 1: B is N x K
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    return int(M), int(N), int(K)


def _mode(mode) -> int:
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"mode must be one of {list(MODES)}")
        return MODES[mode]
    return int(mode)


def gemm_run(A, B, C, plan: Plan, mode="dynamic", stream=None) -> None:
    """gemm_run: enqueue C = A.B (A: M x K bf16, B: K x N bf16, C: M x N fp32); with a plan of
    b_layout 1, B is N x K and C = A.B^T."""
    M, N, K = _check_operands(A, B, C, int(plan.desc.b_layout))
    st = load_library().gemm_run(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                 ctypes.c_void_p(C.data_ptr()), M, N, K, _mode(mode), plan.handle,
                                 ctypes.c_void_p(_stream_ptr(stream)))
    _check(st, "gemm_run", plan)


def gemm_run_raw(A_ptr: int, B_ptr: int, C_ptr: int, M: int, N: int, K: int, plan: Plan, mode="dynamic",
                 stream=None) -> int:
    """gemm_run with raw device pointers; returns the status without raising (ABI tests)."""
    return int(load_library().gemm_run(ctypes.c_void_p(A_ptr), ctypes.c_void_p(B_ptr), ctypes.c_void_p(C_ptr),
                                       int(M), int(N), int(K), _mode(mode),
                                       plan.handle if plan is not None else None,
                                       ctypes.c_void_p(_stream_ptr(stream))))


def gemm_run_noalloc(A, B, C, mode="dynamic", status=None, stream=None) -> None:
    """gemm_run_noalloc: C = A.B with the default 256 x 256 configuration and no plan; the library
    allocates nothing (its scheduler state is a fixed device array). status: optional int32/uint32
    device tensor of one element that receives device error bits."""
    M, N, K = _check_operands(A, B, C, 0)
    sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p()
    st = load_library().gemm_run_noalloc(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                         ctypes.c_void_p(C.data_ptr()), M, N, K, _mode(mode), sp,
                                         ctypes.c_void_p(_stream_ptr(stream)))
    _check(st, "gemm_run_noalloc")


def gemm_run_grouped(As: Sequence, Bs: Sequence, Cs: Sequence, plan: Plan, mode="dynamic", stream=None) -> None:
    """gemm_run_grouped: all problems C_g = A_g.B_g in one launch.

    For many small problems of uneven K, a plan made with group_order=1 (longest
    K first) and claim_policy=2 (contiguous XCD regions, so each XCD runs whole
    problems and shares their operand panels in its own L2) gave the shortest
    dynamic makespan measured on 64 problems of 1024 x 1024 with K from 512 to 8192."""
    G = len(As)
    if not (len(Bs) == len(Cs) == G) or G == 0:
        raise ValueError("need equally many A, B, C (at least one)")
    dims = [_check_operands(a, b, c, int(plan.desc.b_layout)) for a, b, c in zip(As, Bs, Cs)]
    VP = ctypes.c_void_p * G
    I64 = ctypes.c_int64 * G
    st = load_library().gemm_run_grouped(
        G, VP(*[a.data_ptr() for a in As]), VP(*[b.data_ptr() for b in Bs]), VP(*[c.data_ptr() for c in Cs]),
        I64(*[d[0] for d in dims]), I64(*[d[1] for d in dims]), I64(*[d[2] for d in dims]),
        _mode(mode), plan.handle, ctypes.c_void_p(_stream_ptr(stream)))
    _check(st, "gemm_run_grouped", plan)


def gemm_read_log(plan: Plan, cap: Optional[int] = None, strict: bool = True) -> np.ndarray:
    """gemm_read_log: synchronise and return the last run's tile log as a structured array."""
    if cap is None:
        cap = max(int(plan.desc.log_capacity), 0)
    buf = (TileRec * max(cap, 1))()
    n = ctypes.c_size_t(0)
    st = load_library().gemm_read_log(plan.handle, buf, cap, ctypes.byref(n))
    if strict:
        _check(st, "gemm_read_log", plan)
    return np.frombuffer(bytes(buf), dtype=TILE_REC_DTYPE, count=max(cap, 1))[: n.value].copy()


def gemm_read_log_status(plan: Plan, cap: Optional[int] = None):
    """Like gemm_read_log but return (status, records) without raising."""
    if cap is None:
        cap = max(int(plan.desc.log_capacity), 0)
    buf = (TileRec * max(cap, 1))()
    n = ctypes.c_size_t(0)
    st = load_library().gemm_read_log(plan.handle, buf, cap, ctypes.byref(n))
    arr = np.frombuffer(bytes(buf), dtype=TILE_REC_DTYPE, count=max(cap, 1))[: n.value].copy()
    return int(st), arr


def gemm_sync(plan: Plan, strict: bool = True) -> int:
    """gemm_sync: wait for the plan's last run and return (strict=False) or raise on (strict=True) the
    device status of every run since the last check (a gate wait that ran out, a ring protocol
    violation). Works with the tile log off."""
    st = int(load_library().gemm_sync(plan.handle))
    if strict:
        _check(st, "gemm_sync", plan)
    return st


def gemm_plan_info_get(plan: Plan) -> dict:
    info = PlanInfo()
    _check(load_library().gemm_plan_info_get(plan.handle, ctypes.byref(info)), "gemm_plan_info_get", plan)
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def gemm_test_preset_counter(plan: Plan, start: int) -> None:
    _check(load_library().gemm_test_preset_counter(plan.handle, int(start)), "gemm_test_preset_counter", plan)


def gemm_test_preset_gate(plan: Plan, held: int) -> None:
    _check(load_library().gemm_test_preset_gate(plan.handle, int(held)), "gemm_test_preset_gate", plan)


class CuMaskStream:
    """A stream restricted to the compute units of a mask (gemm_test_stream_cu_mask). `torch_stream` is
    the same stream as a torch.cuda.ExternalStream, for events and for the binding's stream arguments."""

    def __init__(self, mask_words: Sequence[int], device: int = 0):
        import torch
        words = [int(w) & 0xFFFFFFFF for w in mask_words]
        arr = (ctypes.c_uint32 * len(words))(*words)
        h = ctypes.c_void_p()
        _check(load_library().gemm_test_stream_cu_mask(ctypes.byref(h), int(device), arr, len(words)),
               "gemm_test_stream_cu_mask")
        self._handle = h
        self.torch_stream = torch.cuda.ExternalStream(h.value, device=torch.device("cuda", int(device)))

    @property
    def cuda_stream(self) -> int:
        return int(self._handle.value or 0)

    def destroy(self) -> None:
        if self._handle:
            self.torch_stream.synchronize()
            _check(load_library().gemm_test_stream_destroy(self._handle), "gemm_test_stream_destroy")
            self._handle = ctypes.c_void_p()


def gemm_test_stream_cu_mask(mask_words: Sequence[int], device: int = 0) -> CuMaskStream:
    return CuMaskStream(mask_words, device)


def gemm_test_stream_destroy(stream: CuMaskStream) -> None:
    stream.destroy()


def gemm_test_spoiler(n_wgs: int, spin_ns: int, stream=None, log=None, wait_resident_ms: float = 0.0,
                      device: int = 0) -> None:
    """gemm_test_spoiler: occupy n_wgs CUs for spin_ns on `stream` (log: uint64 device tensor of 4*n_wgs)."""
    log_ptr = ctypes.c_void_p(log.data_ptr()) if log is not None else ctypes.c_void_p()
    st = load_library().gemm_test_spoiler(int(device), int(n_wgs), int(spin_ns), ctypes.c_void_p(_stream_ptr(stream)),
                                          log_ptr, float(wait_resident_ms))
    _check(st, "gemm_test_spoiler")


def gemm_mfma_probe(iters: int = 20000, random_operands: bool = True, mfma_block: int = 16, device: int = 0) -> dict:
    """gemm_mfma_probe: MFMA-only bf16 rate and shader clock on every CU (no memory traffic), with
    16 x 16 x 32 (mfma_block=16) or 32 x 32 x 16 (mfma_block=32) MFMAs."""
    tf = ctypes.c_double(0.0)
    ghz = ctypes.c_double(0.0)
    st = load_library().gemm_mfma_probe(int(device), int(iters), 1 if random_operands else 0, int(mfma_block),
                                        ctypes.byref(tf), ctypes.byref(ghz))
    _check(st, "gemm_mfma_probe")
    return {"tflops": tf.value, "clock_ghz": ghz.value}


def gemm_hbm_probe(bytes_: int = 1 << 30, kind: str = "read", reps: int = 20, device: int = 0) -> float:
    """gemm_hbm_probe: GB/s a plain streaming kernel reaches ('read': read once; 'copy': read + write)."""
    gbs = ctypes.c_double(0.0)
    st = load_library().gemm_hbm_probe(int(device), int(bytes_), {"read": 0, "copy": 1}[kind], int(reps),
                                       ctypes.byref(gbs))
    _check(st, "gemm_hbm_probe")
    return gbs.value


def bf16_from_bits(bits: np.ndarray, device="cuda"):
    """Upload uint16 bf16 bit patterns as a torch.bfloat16 device tensor (bits unchanged)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def gemm(A, B, C=None, mode="dynamic", plan: Optional[Plan] = None, stream=None):
    """C = A.B through gemm_run (A: M x K bf16, B: K x N bf16; with a plan of b_layout 1, B is N x K).

    C (optional) is an M x N float32 device tensor to overwrite; it is allocated when absent. The run goes on
    `stream` (default: the current stream). With no plan, a default 256 x 256 plan is made for the call, the
    call waits for the run and raises PtgError on a device-side failure too; with a caller's plan it returns
    at once (check the plan with gemm_sync). Returns C."""
    import torch
    own = plan is None
    if own:
        plan = gemm_create()
    try:
        n = B.shape[1] if int(plan.desc.b_layout) == 0 else B.shape[0]
        if C is None:
            C = torch.empty((A.shape[0], n), dtype=torch.float32, device=A.device)
        gemm_run(A, B, C, plan, mode=mode, stream=stream)
        if own:
            gemm_sync(plan)
    finally:
        if own:
            plan.destroy()
    return C


def matmul(A, B, mode="dynamic", plan: Optional[Plan] = None, stream=None):
    """Convenience: allocate C and run C = A.B with a default 256x256 plan."""
    import torch
    own = plan is None
    if own:
        plan = gemm_create()
    n = B.shape[1] if int(plan.desc.b_layout) == 0 else B.shape[0]
    C = torch.empty((A.shape[0], n), dtype=torch.float32, device=A.device)
    try:
        gemm_run(A, B, C, plan, mode=mode, stream=stream)
        if own:
            gemm_sync(plan)  # waits for the run and raises on a device-side failure
    finally:
        if own:
            plan.destroy()
    return C

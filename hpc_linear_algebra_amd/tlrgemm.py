"""ctypes binding of libtlrgemm.so (include/tlrgemm.h), same names as the C ABI.

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  The library must have been built (hpc_linear_algebra_amd.build);
there is no fallback of any kind, and loading fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from typing import List, Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtlrgemm.so")

TLR_OK, TLR_ERR_INVALID_ARG, TLR_ERR_RANK, TLR_ERR_WORKSPACE = 0, -1, -2, -3
TLR_ERR_UNSUPPORTED, TLR_ERR_HIP, TLR_ERR_NOT_BOUND = -4, -5, -6
TLR_F32, TLR_F64, TLR_F16, TLR_BF16 = 0, 1, 2, 3
TLR_OP_N, TLR_OP_T = 0, 1
TLR_ORDER_RIGHT, TLR_ORDER_LEFT = 0, 1
TLR_PLAN_FORCE_RIGHT, TLR_PLAN_FORCE_LEFT, TLR_PLAN_NO_REGIONS, TLR_PLAN_VALIDATE = 0x1, 0x2, 0x4, 0x8
TLR_PLAN_PIPELINE = 0x10
TLR_PLAN_PER_K = 0x20
TLR_STATIC_WORKSPACE_BYTES = 256 * 1024 * 1024

EXPORTED = [
    "tlr_gemm_analyze", "tlr_gemm_workspace_bytes", "tlr_plan_info", "tlr_plan_rect",
    "tlr_plan_stage_shapes", "tlr_plan_launch", "tlr_plan_destroy", "tlr_plan_bind",
    "tlr_gemm_execute", "tlr_gemm_execute_noalloc", "tlr_expand", "tlr_compress_workspace_bytes",
    "tlr_compress", "tlr_compress_profile", "tlr_compress_profile_read", "tlr_plan_profile",
    "tlr_plan_profile_read", "tlr_dense_gemm",
    "tlr_status_string", "tlr_last_error", "tlr_version",
]


class tlr_shape(ctypes.Structure):
    _fields_ = [("rows", c_int64), ("cols", c_int64), ("b", c_int32), ("has_diag", c_int32),
                ("ranks", POINTER(c_int32))]


class tlr_buffers(ctypes.Structure):
    _fields_ = [("diag", c_void_p), ("outer", c_void_p), ("inner", c_void_p)]


class tlr_plan_summary(ctypes.Structure):
    _fields_ = [("m", c_int64), ("n", c_int64), ("k", c_int64),
                ("useful_flops", c_double), ("executed_flops", c_double),
                ("flops_right", c_double), ("flops_left", c_double),
                ("final_flops_right", c_double), ("final_flops_left", c_double),
                ("algorithmic_bytes", c_double),
                ("workspace_bytes", c_size_t), ("descriptor_bytes", c_size_t),
                ("runs", c_int32), ("groups", c_int32), ("launches", c_int32), ("dtype", c_int32)]


class TLRError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_lib = None


def lib():
    """Load libtlrgemm.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m hpc_linear_algebra_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    L.tlr_gemm_analyze.argtypes = [c_int32, c_int32, POINTER(tlr_shape), c_int32, POINTER(tlr_shape),
                                   c_int64, c_int64, c_int64, c_int64, c_size_t, c_int32, c_uint32,
                                   POINTER(P)]
    L.tlr_gemm_workspace_bytes.argtypes = [c_int32, c_int32, POINTER(tlr_shape), c_int32, POINTER(tlr_shape),
                                           c_int64, c_int64, c_int32, c_uint32, c_int32, POINTER(c_size_t)]
    L.tlr_plan_info.argtypes = [P, POINTER(tlr_plan_summary)]
    L.tlr_plan_rect.argtypes = [P, c_int32, POINTER(c_int32), POINTER(c_size_t), POINTER(c_double)]
    L.tlr_plan_stage_shapes.argtypes = [P, c_int32, c_int32, POINTER(c_int64), c_int32, POINTER(c_int32)]
    L.tlr_plan_launch.argtypes = [P, c_int32, POINTER(c_int32), POINTER(c_double)]
    L.tlr_plan_destroy.argtypes = [P]
    L.tlr_plan_bind.argtypes = [P, P, c_size_t, P]
    L.tlr_gemm_execute.argtypes = [P, c_double, POINTER(tlr_buffers), POINTER(tlr_buffers), P, c_int64,
                                   c_double, P, c_int64, P, c_size_t, POINTER(P), c_int32]
    L.tlr_gemm_execute_noalloc.argtypes = [P, c_double, POINTER(tlr_buffers), POINTER(tlr_buffers), P, c_int64,
                                           c_double, P, c_int64, POINTER(P), c_int32]
    L.tlr_expand.argtypes = [c_int32, c_int64, c_int64, c_int32, c_int32, P, POINTER(tlr_buffers), c_double,
                             c_double, P, c_int64, P, c_size_t, P]
    L.tlr_compress_workspace_bytes.argtypes = [c_int32, c_int64, c_int64, c_int32, c_int32, POINTER(c_size_t)]
    L.tlr_compress.argtypes = [c_int32, c_int64, c_int64, c_int32, c_int32, P, c_int64, c_double, c_int32, P, P,
                               P, P, P, c_int64, P, P, c_size_t, P]
    L.tlr_compress_profile.argtypes = [c_int32]
    L.tlr_compress_profile_read.argtypes = [POINTER(c_double), POINTER(c_int32)]
    L.tlr_plan_profile.argtypes = [P, c_int32]
    L.tlr_plan_profile_read.argtypes = [P, POINTER(c_double), POINTER(c_double), POINTER(c_int32)]
    L.tlr_dense_gemm.argtypes = [c_int32, c_int32, c_int32, c_int64, c_int64, c_int64, c_double, P, c_int64,
                                 P, c_int64, c_double, P, c_int64, P]
    for name in EXPORTED[:-3]:
        getattr(L, name).restype = c_int32
    L.tlr_status_string.argtypes = [c_int32]
    L.tlr_status_string.restype = c_char_p
    L.tlr_last_error.argtypes = []
    L.tlr_last_error.restype = c_char_p
    L.tlr_version.argtypes = []
    L.tlr_version.restype = c_char_p
    _lib = L
    return L


def _check(st: int, where: str):
    if st != TLR_OK:
        L = lib()
        raise TLRError(st, where, f"{L.tlr_status_string(st).decode()}: {L.tlr_last_error().decode()}")


def _op(x) -> int:
    if x in ("N", TLR_OP_N):
        return TLR_OP_N
    if x in ("T", TLR_OP_T):
        return TLR_OP_T
    raise ValueError(f"bad op {x!r}")


def _dt(x) -> int:
    if x in ("f64", TLR_F64, np.float64):
        return TLR_F64
    if x in ("f32", TLR_F32, np.float32):
        return TLR_F32
    if x in ("f16", TLR_F16, np.float16):
        return TLR_F16
    if x in ("bf16", TLR_BF16):
        return TLR_BF16
    raise ValueError(f"bad dtype {x!r}")


class Shape:
    """Host description of one stored TLR operand (keeps its rank array alive)."""

    def __init__(self, rows: int, cols: int, b: int, ranks: np.ndarray, has_diag: bool):
        R = np.asarray(ranks, dtype=np.int32)
        self.ranks_cm = np.ascontiguousarray(R.T).ravel()      # column-major r[i + j*qr]
        self.c = tlr_shape(rows, cols, b, 1 if has_diag else 0,
                           self.ranks_cm.ctypes.data_as(POINTER(c_int32)))


class Plan:
    """Owns a tlr_plan handle."""

    def __init__(self, handle: int, keep):
        self.h = c_void_p(handle)
        self._keep = keep

    def __del__(self):
        if getattr(self, "h", None) and self.h.value and _lib is not None:
            _lib.tlr_plan_destroy(self.h)
            self.h = c_void_p(0)


def tlr_gemm_analyze(dtype, opA, A: Optional[Shape], opB, B: Optional[Shape], dense_rows: int = 0,
                     dense_cols: int = 0, ldb: int = 0, ldc: int = 0, workspace_budget: int = 0,
                     n_streams: int = 1, flags: int = 0) -> Plan:
    """A or B None: that operand is dense (stored dense_rows x dense_cols, leading dim ldb)."""
    L = lib()
    h = c_void_p()
    st = L.tlr_gemm_analyze(_dt(dtype), _op(opA), ctypes.byref(A.c) if A is not None else None, _op(opB),
                            ctypes.byref(B.c) if B is not None else None, dense_rows, dense_cols, ldb, ldc,
                            workspace_budget, n_streams, flags, ctypes.byref(h))
    _check(st, "tlr_gemm_analyze")
    return Plan(h.value, (A, B))


def tlr_gemm_workspace_bytes(dtype, opA, A: Optional[Shape], opB, B: Optional[Shape], dense_rows: int = 0,
                             dense_cols: int = 0, n_streams: int = 1, flags: int = 0, runs: int = 1) -> int:
    L = lib()
    out = c_size_t()
    st = L.tlr_gemm_workspace_bytes(_dt(dtype), _op(opA), ctypes.byref(A.c) if A is not None else None, _op(opB),
                                    ctypes.byref(B.c) if B is not None else None, dense_rows, dense_cols,
                                    n_streams, flags, runs, ctypes.byref(out))
    _check(st, "tlr_gemm_workspace_bytes")
    return int(out.value)


def tlr_plan_info(p: Plan) -> dict:
    s = tlr_plan_summary()
    _check(lib().tlr_plan_info(p.h, ctypes.byref(s)), "tlr_plan_info")
    return {f: getattr(s, f) for f, _ in tlr_plan_summary._fields_}


def tlr_plan_rect(p: Plan, idx: int) -> dict:
    o = (c_int32 * 6)()
    ws = c_size_t()
    fl = c_double()
    _check(lib().tlr_plan_rect(p.h, idx, o, ctypes.byref(ws), ctypes.byref(fl)), "tlr_plan_rect")
    return dict(i0=o[0], i1=o[1], j0=o[2], j1=o[3], order=o[4], group=o[5], ws_bytes=int(ws.value),
                useful_flops=fl.value)


def tlr_plan_stage_shapes(p: Plan, rect: int, stage: int) -> List[tuple]:
    cnt = c_int32()
    _check(lib().tlr_plan_stage_shapes(p.h, rect, stage, None, 0, ctypes.byref(cnt)), "tlr_plan_stage_shapes")
    n = cnt.value
    buf = (c_int64 * (3 * max(n, 1)))()
    _check(lib().tlr_plan_stage_shapes(p.h, rect, stage, buf, n, ctypes.byref(cnt)), "tlr_plan_stage_shapes")
    return [(buf[3 * t], buf[3 * t + 1], buf[3 * t + 2]) for t in range(n)]


def tlr_plan_launch(p: Plan, idx: int) -> dict:
    oi = (c_int32 * 4)()
    of = (c_double * 2)()
    _check(lib().tlr_plan_launch(p.h, idx, oi, of), "tlr_plan_launch")
    return dict(stage=oi[0], tasks=oi[1], workgroups=oi[2], group=oi[3], useful_flops=of[0],
                executed_flops=of[1])


def tlr_plan_bind(p: Plan, dev_desc: int, nbytes: int, stream: int = 0):
    _check(lib().tlr_plan_bind(p.h, c_void_p(dev_desc), nbytes, c_void_p(stream)), "tlr_plan_bind")


def buffers(diag: int = 0, outer: int = 0, inner: int = 0) -> tlr_buffers:
    return tlr_buffers(c_void_p(diag or None), c_void_p(outer or None), c_void_p(inner or None))


def tlr_gemm_execute(p: Plan, alpha: float, A: Optional[tlr_buffers], B: Optional[tlr_buffers], B_dense: int,
                     ldb: int, beta: float, C: int, ldc: int, workspace: int, workspace_bytes: int,
                     streams: Sequence[int]):
    """B_dense / ldb: the dense operand (A's storage when A is None, else B's)."""
    arr = (c_void_p * max(1, len(streams)))(*[c_void_p(s or None) for s in streams])
    st = lib().tlr_gemm_execute(p.h, alpha, ctypes.byref(A) if A is not None else None,
                                ctypes.byref(B) if B is not None else None,
                                c_void_p(B_dense or None), ldb, beta, c_void_p(C or None), ldc,
                                c_void_p(workspace or None), workspace_bytes, arr, max(1, len(streams)))
    _check(st, "tlr_gemm_execute")


def tlr_gemm_execute_noalloc(p: Plan, alpha: float, A: Optional[tlr_buffers], B: Optional[tlr_buffers],
                             B_dense: int, ldb: int, beta: float, C: int, ldc: int, streams: Sequence[int]):
    """tlr_gemm_execute with the library's static device workspace (no workspace argument)."""
    arr = (c_void_p * max(1, len(streams)))(*[c_void_p(s or None) for s in streams])
    st = lib().tlr_gemm_execute_noalloc(p.h, alpha, ctypes.byref(A) if A is not None else None,
                                        ctypes.byref(B) if B is not None else None,
                                        c_void_p(B_dense or None), ldb, beta, c_void_p(C or None), ldc, arr,
                                        max(1, len(streams)))
    _check(st, "tlr_gemm_execute_noalloc")


def tlr_expand(dtype, rows: int, cols: int, b: int, has_diag: bool, ranks_dev: int, X: tlr_buffers, alpha: float,
               beta: float, C: int, ldc: int, workspace: int, workspace_bytes: int, stream: int = 0):
    st = lib().tlr_expand(_dt(dtype), rows, cols, b, 1 if has_diag else 0, c_void_p(ranks_dev or None),
                          ctypes.byref(X), alpha, beta, c_void_p(C or None), ldc, c_void_p(workspace or None),
                          workspace_bytes, c_void_p(stream or None))
    _check(st, "tlr_expand")


def tlr_compress_workspace_bytes(dtype, rows: int, cols: int, b: int, max_rank: int) -> int:
    out = c_size_t()
    _check(lib().tlr_compress_workspace_bytes(_dt(dtype), rows, cols, b, max_rank, ctypes.byref(out)),
           "tlr_compress_workspace_bytes")
    return int(out.value)


def tlr_compress(dtype, rows: int, cols: int, b: int, has_diag: bool, X: int, ldx: int, tol: float, max_rank: int,
                 omega: int, ranks_out: int, diag: int, outer: int, inner: int, capacity: int, info: int,
                 workspace: int, workspace_bytes: int, stream: int = 0):
    st = lib().tlr_compress(_dt(dtype), rows, cols, b, 1 if has_diag else 0, c_void_p(X or None), ldx, tol, max_rank,
                            c_void_p(omega or None), c_void_p(ranks_out or None), c_void_p(diag or None),
                            c_void_p(outer or None), c_void_p(inner or None), capacity, c_void_p(info or None),
                            c_void_p(workspace or None), workspace_bytes, c_void_p(stream or None))
    _check(st, "tlr_compress")


COMPRESS_PROFILE_GROUPS = ("tile norms", "sketch products", "QR of the sketches", "projections",
                           "QR of the projections", "Jacobi SVD and ranks", "factor products", "rank scan",
                           "packing")


def tlr_compress_profile(max_calls: int):
    _check(lib().tlr_compress_profile(max_calls), "tlr_compress_profile")


def tlr_compress_profile_read():
    """(milliseconds per kernel group summed over the recorded calls, calls)."""
    ms = (c_double * len(COMPRESS_PROFILE_GROUPS))()
    calls = c_int32()
    _check(lib().tlr_compress_profile_read(ms, ctypes.byref(calls)), "tlr_compress_profile_read")
    return list(ms), calls.value


def tlr_plan_profile(p: Plan, max_executes: int):
    _check(lib().tlr_plan_profile(p.h, max_executes), "tlr_plan_profile")


def tlr_plan_profile_read(p: Plan, launches: int):
    st_ms = (c_double * 5)()
    l_ms = (c_double * max(1, launches))()
    ex = c_int32()
    _check(lib().tlr_plan_profile_read(p.h, st_ms, l_ms, ctypes.byref(ex)), "tlr_plan_profile_read")
    return list(st_ms), list(l_ms)[:launches], ex.value


def tlr_dense_gemm(dtype, opA, opB, m: int, n: int, k: int, alpha: float, A: int, lda: int, B: int,
                   ldb: int, beta: float, C: int, ldc: int, stream: int = 0):
    st = lib().tlr_dense_gemm(_dt(dtype), _op(opA), _op(opB), m, n, k, alpha, c_void_p(A or None), lda,
                              c_void_p(B or None), ldb, beta, c_void_p(C or None), ldc, c_void_p(stream or None))
    _check(st, "tlr_dense_gemm")


def tlr_status_string(s: int) -> str:
    return lib().tlr_status_string(s).decode()


def tlr_last_error() -> str:
    return lib().tlr_last_error().decode()


def tlr_version() -> str:
    return lib().tlr_version().decode()

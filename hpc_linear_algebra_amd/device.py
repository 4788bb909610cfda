"""PyTorch plumbing around the C ABI: device copies of packed operands and a
plan object that owns its descriptor and workspace buffers.

torch is used only for device memory and streams.  A column-major m x n
matrix with leading dimension ld is a contiguous torch tensor of shape
(n, ld); element (r, c) is tensor[c, r].
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import layout
from . import tlrgemm as T
from tlr_inputs import TLRTiles

_TORCH = {"f64": torch.float64, "f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _dev(x: Optional[np.ndarray], device, dtype: str) -> Optional[torch.Tensor]:
    if x is None or x.size == 0:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=_TORCH[dtype])


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


class DeviceTLR:
    """A TLR operand packed on the host and copied to the GPU.  For the 16-bit
    types the stored ranks are the logical ranks rounded up to a multiple of 8
    (zero factor columns); ``logical_ranks`` keeps the originals."""

    def __init__(self, t: TLRTiles, device="cuda"):
        self.logical_ranks = np.asarray(t.ranks, dtype=np.int32)
        if t.dtype in layout.SIXTEEN_BIT:
            t = layout.round_ranks(t, 8)
        pk = layout.pack(t)
        self.rows, self.cols, self.b = t.rows, t.cols, t.b
        self.dtype = t.dtype
        self.has_diag = t.has_diag
        self.ranks = np.asarray(t.ranks, dtype=np.int32)
        self.shape = T.Shape(t.rows, t.cols, t.b, self.ranks, t.has_diag)
        self.outer = _dev(pk["outer"], device, t.dtype)
        self.inner = _dev(pk["inner"], device, t.dtype)
        self.diag = _dev(pk["diag"], device, t.dtype)

    def buffers(self) -> T.tlr_buffers:
        return T.buffers(_ptr(self.diag), _ptr(self.outer), _ptr(self.inner))

    def ranks_device(self) -> torch.Tensor:
        """The stored ranks as a device int32 array, column-major q_r x q_c (as
        tlr_expand reads them)."""
        if getattr(self, "_ranks_dev", None) is None:
            cm = np.ascontiguousarray(self.ranks.T).ravel().astype(np.int32)
            self._ranks_dev = torch.from_numpy(cm).to(self.outer.device if self.outer is not None else "cuda")
        return self._ranks_dev


def dense_to_device(M: np.ndarray, device="cuda", ld: Optional[int] = None,
                    dtype: Optional[str] = None) -> torch.Tensor:
    """Column-major device copy: tensor of shape (cols, ld), of element type
    ``dtype`` (default: the array's own)."""
    rows, cols = M.shape
    ld = rows if ld is None else ld
    t = torch.from_numpy(layout.to_colmajor(M, ld).reshape(cols, ld))
    return t.to(device) if dtype is None else t.to(device=device, dtype=_TORCH[dtype])


def dense_from_device(t: torch.Tensor, rows: int, cols: int) -> np.ndarray:
    """Host copy as a [row, col] array (16-bit values widened to float32)."""
    t = t.detach()
    if t.dtype in (torch.float16, torch.bfloat16):
        t = t.float()
    return t.cpu().numpy()[:, :rows].T


class TLRGemm:
    """Analyse, allocate descriptor + workspace tensors, bind; then execute.

    Either A or B may be a dense operand (None at construction, with its
    stored dense_shape and leading dimension ldb; its device tensor is passed
    in that position at call time)."""

    def __init__(self, dtype: str, opA: str, A: Optional[DeviceTLR], opB: str, B, ldc: int,
                 dense_shape: Optional[tuple] = None, ldb: int = 0, budget: int = 0,
                 n_streams: int = 1, flags: int = 0, device="cuda"):
        self.dtype = dtype
        self.dense_a = A is None
        self.dense = B is None
        dr, dc = dense_shape if (self.dense or self.dense_a) else (0, 0)
        self.plan = T.tlr_gemm_analyze(dtype, opA, None if self.dense_a else A.shape, opB,
                                       None if self.dense else B.shape, dr, dc, ldb, ldc, budget, n_streams,
                                       flags)
        self.info = T.tlr_plan_info(self.plan)
        self.ldb, self.ldc = ldb, ldc
        self.desc = torch.empty(self.info["descriptor_bytes"], dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(self.info["workspace_bytes"], 256), dtype=torch.uint8, device=device)
        T.tlr_plan_bind(self.plan, self.desc.data_ptr(), self.desc.numel(),
                        torch.cuda.current_stream().cuda_stream)

    def rects(self):
        return [T.tlr_plan_rect(self.plan, r) for r in range(self.info["runs"])]

    def launches(self):
        return [T.tlr_plan_launch(self.plan, l) for l in range(self.info["launches"])]

    def __call__(self, alpha: float, A, B, beta: float, C: torch.Tensor,
                 streams: Optional[Sequence[int]] = None):
        if streams is None:
            streams = [torch.cuda.current_stream().cuda_stream]
        Ab, Bb, Dd = None, None, 0
        if self.dense_a:
            Dd, Bb = A.data_ptr(), B.buffers()
        elif self.dense:
            Ab, Dd = A.buffers(), B.data_ptr()
        else:
            Ab, Bb = A.buffers(), B.buffers()
        T.tlr_gemm_execute(self.plan, alpha, Ab, Bb, Dd, self.ldb, beta, C.data_ptr(), self.ldc,
                           self.ws.data_ptr(), self.ws.numel(), list(streams))
        return C


class TLROutputGemm:
    """C <- alpha op(A) op(B) + beta C with C in TLR format, every off-diagonal
    result tile truncated to a relative Frobenius tolerance, the diagonal kept
    dense.  Three library calls on one stream: tlr_expand of C into a dense
    scratch (skipped when beta == 0), tlr_gemm_execute into that scratch, and
    tlr_compress of it into the result buffers (device ranks, diagonal slots,
    packed factors with room for ``capacity`` columns, info[5])."""

    def __init__(self, dtype: str, opA: str, A: DeviceTLR, opB: str, B: DeviceTLR, b: int, has_diag: bool,
                 max_rank: int, capacity: Optional[int] = None, budget: int = 0, device="cuda"):
        self.dtype = dtype
        self.gemm = TLRGemm(dtype, opA, A, opB, B, ldc=(A.rows if opA == "N" else A.cols), budget=budget,
                            device=device)
        self.m = self.gemm.info["m"]
        self.n = self.gemm.info["n"]
        self.b, self.has_diag, self.max_rank = b, has_diag, max_rank
        self.qr, self.qc = -(-self.m // b), -(-self.n // b)
        nt = self.qr * self.qc
        n_off = nt - (min(self.qr, self.qc) if has_diag else 0)
        self.capacity = n_off * max_rank if capacity is None else capacity
        tdt = _TORCH[dtype]
        self.scratch = torch.empty((self.n, self.m), dtype=tdt, device=device)     # column-major m x n
        self.ews = torch.empty(max(16 * nt, 256), dtype=torch.uint8, device=device)
        self.cws = torch.empty(T.tlr_compress_workspace_bytes(dtype, self.m, self.n, b, max_rank),
                               dtype=torch.uint8, device=device)
        self.ranks = torch.zeros(nt, dtype=torch.int32, device=device)
        self.diag = torch.zeros((max(1, self.qr) * b * b) if has_diag else 1, dtype=tdt, device=device)
        self.outer = torch.zeros(max(1, self.capacity) * b, dtype=tdt, device=device)
        self.inner = torch.zeros(max(1, self.capacity) * b, dtype=tdt, device=device)
        self.info = torch.zeros(6, dtype=torch.int32, device=device)

    def __call__(self, alpha: float, A: DeviceTLR, B: DeviceTLR, beta: float, C: Optional[DeviceTLR], tol: float,
                 omega: torch.Tensor, stream: Optional[int] = None):
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        if beta != 0.0:
            T.tlr_expand(self.dtype, self.m, self.n, self.b, self.has_diag, C.ranks_device().data_ptr(), C.buffers(),
                         1.0, 0.0, self.scratch.data_ptr(), self.m, self.ews.data_ptr(), self.ews.numel(), s)
        self.gemm(alpha, A, B, beta, self.scratch, [s])
        T.tlr_compress(self.dtype, self.m, self.n, self.b, self.has_diag, self.scratch.data_ptr(), self.m, tol,
                       self.max_rank, omega.data_ptr(), self.ranks.data_ptr(), _ptr(self.diag) if self.has_diag else 0,
                       self.outer.data_ptr(), self.inner.data_ptr(), self.capacity, self.info.data_ptr(),
                       self.cws.data_ptr(), self.cws.numel(), s)
        return self

    def host_result(self):
        """(ranks q_r x q_c, outer, inner, diag, info) copied to the host
        (after the caller has synchronised)."""
        R = self.ranks.cpu().numpy().reshape(self.qc, self.qr).T.copy()
        return (R, self.outer.cpu().numpy(), self.inner.cpu().numpy(),
                self.diag.cpu().numpy() if self.has_diag else None, self.info.cpu().numpy())

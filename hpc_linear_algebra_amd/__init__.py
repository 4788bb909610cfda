"""Tile-Low-Rank GEMM on AMD Instinct MI355X (gfx950).

C <- alpha op(A) op(B) + beta C with dense C and A, B or both stored as
Tile-Low-Rank matrices, in float64, float32, half or bfloat16, computed by
hand-written HIP/MFMA kernels behind the C ABI in include/tlrgemm.h.

  tlrgemm   ctypes binding of libtlrgemm.so (same names as the C ABI)
  layout    host packing of per-tile data into the library's buffer layout
  device    torch plumbing: device buffers, plan with descriptor + workspace
  build     compiles libtlrgemm.so in-tree for gfx950
"""
from . import tlrgemm, layout  # noqa: F401

__all__ = ["tlrgemm", "layout"]

"""Packing of per-tile TLR data into the library's buffers, and column-major
helpers for dense matrices.

Packing rules ("Tile-Low-Rank GEMM: Designing Storage Around the
Contraction", "Packing for the contraction"): outer factors U packed by tile
row, inner factors V by tile column, each column-major with leading dimension
b, each tile taking exactly its rank's worth of columns; dense diagonal tiles
in b x b column-major slots.  This is input preparation on the host: the
product itself runs only in the HIP library.

A column-major m x n matrix with leading dimension ld is held in a flat array
``buf`` with element (r, c) at ``buf[r + c*ld]``.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from tlr_inputs import TLRTiles


def _np(dtype: str):
    # 16-bit element types are held in float32 host arrays (values on the
    # 16-bit grid) and converted when copied to the device
    return np.float64 if dtype == "f64" else np.float32


SIXTEEN_BIT = ("f16", "bf16")


def round_ranks(t: TLRTiles, multiple: int = 8) -> TLRTiles:
    """The operand with every stored rank rounded up to a multiple of
    ``multiple`` by appending zero factor columns (section "Packing for the
    contraction": on the 16-bit paths each stored rank is a multiple of 8, so
    every factor column offset is a multiple of 16 bytes; the logical rank, and
    the matrix, are unchanged).  A rank never exceeds its tile's smaller side,
    so that side must itself be a multiple of ``multiple`` wherever a rank is
    rounded."""
    U, V = {}, {}
    R = np.array(t.ranks, dtype=np.int32, copy=True)
    rs, cs = t.row_sizes, t.col_sizes
    for (i, j), u in t.U.items():
        v = t.V[(i, j)]
        r = u.shape[1]
        want = -(-r // multiple) * multiple
        if want > min(rs[i], cs[j]):
            raise ValueError(f"tile ({i},{j}): rank {r} cannot be rounded up to {want}")
        if want > r:
            u = np.concatenate([u, np.zeros((u.shape[0], want - r), u.dtype)], axis=1)
            v = np.concatenate([v, np.zeros((v.shape[0], want - r), v.dtype)], axis=1)
        U[(i, j)], V[(i, j)] = u, v
        R[i, j] = want
    return TLRTiles(t.rows, t.cols, t.b, R, t.diag, U, V, t.dtype)


def pack(t: TLRTiles) -> Dict[str, Optional[np.ndarray]]:
    """Flat outer / inner / diag buffers and the column-major rank array."""
    b = t.b
    rs, cs = t.row_sizes, t.col_sizes
    qr, qc = len(rs), len(cs)
    R = np.asarray(t.ranks, dtype=np.int64)
    total = int(R.sum())
    dt = _np(t.dtype)
    outer = np.zeros((max(total, 0), b), dtype=dt)     # row c of this array = column c of the buffer
    inner = np.zeros((max(total, 0), b), dtype=dt)
    col = 0
    for i in range(qr):
        for j in range(qc):
            r = int(R[i, j])
            if r:
                outer[col:col + r, :rs[i]] = t.U[(i, j)].T
            col += r
    col = 0
    for j in range(qc):
        for i in range(qr):
            r = int(R[i, j])
            if r:
                inner[col:col + r, :cs[j]] = t.V[(i, j)].T
            col += r
    diag = None
    if t.has_diag:
        d = np.zeros((qr, b, b), dtype=dt)
        for i in range(qr):
            d[i, :rs[i], :rs[i]] = np.asarray(t.diag[i]).T
        diag = d.ravel()
    return dict(outer=outer.ravel(), inner=inner.ravel(), diag=diag,
                ranks=np.ascontiguousarray(R.T.astype(np.int32)).ravel())


def to_colmajor(M: np.ndarray, ld: Optional[int] = None) -> np.ndarray:
    """Flat column-major copy of a 2-D array (leading dimension ld >= rows)."""
    rows, cols = M.shape
    ld = rows if ld is None else ld
    out = np.zeros((cols, ld), dtype=M.dtype)
    out[:, :rows] = M.T
    return out.ravel()


def from_colmajor(buf: np.ndarray, rows: int, cols: int, ld: Optional[int] = None) -> np.ndarray:
    ld = rows if ld is None else ld
    return np.asarray(buf).reshape(cols, ld)[:, :rows].T

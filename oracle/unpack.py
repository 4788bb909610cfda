"""Read packed TLR buffers back into tiles, from the packing rules alone.

Follows "Tile-Low-Rank GEMM: Designing Storage Around the Contraction",
section "Packing for the contraction": outer factors (U) are packed by tile
row and inner factors (V) by tile column, each factor column-major, each tile
taking exactly r_ij columns; the offset of tile k inside row panel i is the
prefix sum p_i(k) of the ranks before it.  Dense diagonal tiles sit in a
3-D array of b x b column-major slots ("TLR Matrix Multiplication", section
"Introduction: TLR GEMM").  The leading dimension of every factor buffer and
diagonal slot is the tile size b.

Flat buffer convention: element (row, col) of a column-major buffer with
leading dimension b is ``buf[row + col * b]``.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from tlr_inputs import TLRTiles, tile_sizes


def _col(buf: np.ndarray, b: int, col: int, nrows: int) -> np.ndarray:
    start = col * b
    return buf[start:start + nrows]


def unpack(rows: int, cols: int, b: int, ranks: np.ndarray, has_diag: bool,
           outer: np.ndarray, inner: np.ndarray, diag: Optional[np.ndarray],
           dtype: str) -> TLRTiles:
    rs, cs = tile_sizes(rows, b), tile_sizes(cols, b)
    qr, qc = len(rs), len(cs)
    R = np.asarray(ranks)
    U: Dict[Tuple[int, int], np.ndarray] = {}
    V: Dict[Tuple[int, int], np.ndarray] = {}
    # outer: walk tile rows in order; inside a row, tiles left to right
    col = 0
    for i in range(qr):
        for j in range(qc):
            if has_diag and i == j:
                continue
            r = int(R[i, j])
            u = np.zeros((rs[i], r), dtype=outer.dtype)
            for a in range(r):
                u[:, a] = _col(outer, b, col + a, rs[i])
            U[(i, j)] = u
            col += r
    # inner: walk tile columns in order; inside a column, tiles top to bottom
    col = 0
    for j in range(qc):
        for i in range(qr):
            if has_diag and i == j:
                continue
            r = int(R[i, j])
            v = np.zeros((cs[j], r), dtype=inner.dtype)
            for a in range(r):
                v[:, a] = _col(inner, b, col + a, cs[j])
            V[(i, j)] = v
            col += r
    D: Optional[List[np.ndarray]] = None
    if has_diag:
        D = []
        for i in range(qr):
            slot = diag[i * b * b:(i + 1) * b * b]
            d = np.zeros((rs[i], rs[i]), dtype=diag.dtype)
            for c in range(rs[i]):
                d[:, c] = slot[c * b:c * b + rs[i]]
            D.append(d)
    return TLRTiles(rows, cols, b, R.astype(np.int32), D, U, V, dtype)

"""Dense definition of the TLR GEMM, in float64 on the CPU.

Follows "Tile-Low-Rank GEMM: Designing Storage Around the Contraction",
introduction (the operation C <- alpha op(A) op(B) + beta C with dense C and
one or both operands TLR) and section "Many small GEMMs" (each off-diagonal
tile equals U_ik V_ik^T); dense diagonal tiles and smaller boundary tiles
follow "TLR Matrix Multiplication", section "Introduction: TLR GEMM".

The method computes this product exactly (up to rounding order), so the
oracle is the definition: rebuild every tile densely, apply op, multiply once.
fp32 inputs are used as stored (already rounded) and upcast to float64.
"""
from __future__ import annotations

import time
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from tlr_inputs import TLRTiles


def offsets(sizes: Sequence[int]) -> List[int]:
    out, acc = [], 0
    for s in sizes:
        out.append(acc)
        acc += s
    return out


def dense_tile(t: TLRTiles, i: int, j: int) -> np.ndarray:
    """Tile (i, j) of the stored matrix as a float64 array."""
    rs, cs = t.row_sizes, t.col_sizes
    if t.has_diag and i == j:
        return np.asarray(t.diag[i], dtype=np.float64)
    r = int(t.ranks[i, j])
    if r == 0:
        return np.zeros((rs[i], cs[j]))
    u = np.asarray(t.U[(i, j)], dtype=np.float64)
    v = np.asarray(t.V[(i, j)], dtype=np.float64)
    return u @ v.T


def reconstruct(t: TLRTiles) -> np.ndarray:
    """The stored matrix as one dense float64 array (rows x cols)."""
    out = np.zeros((t.rows, t.cols))
    ro, co = offsets(t.row_sizes), offsets(t.col_sizes)
    for i, s in enumerate(t.row_sizes):
        for j, w in enumerate(t.col_sizes):
            out[ro[i]:ro[i] + s, co[j]:co[j] + w] = dense_tile(t, i, j)
    return out


def _op(M: np.ndarray, op: str) -> np.ndarray:
    if op == "N":
        return M
    if op == "T":
        return M.T
    raise ValueError(op)


def gemm_reference(alpha: float, opA: str, A, opB: str, B,
                   beta: float, C_in: Optional[np.ndarray]) -> np.ndarray:
    """alpha op(A) op(B) + beta C_in in float64; C_in is never read when beta == 0.

    ``A`` and ``B`` are each a TLRTiles or a dense 2-D array (the TLR x dense
    and dense x TLR products, both within the pages' "one or both operands in
    TLR format")."""
    Ad = reconstruct(A) if isinstance(A, TLRTiles) else np.asarray(A, dtype=np.float64)
    Ad = _op(Ad, opA)
    Bd = reconstruct(B) if isinstance(B, TLRTiles) else np.asarray(B, dtype=np.float64)
    Bd = _op(Bd, opB)
    if Ad.shape[1] != Bd.shape[0]:
        raise ValueError("inner dimensions differ")
    out = alpha * (Ad @ Bd)
    if beta != 0.0:
        out = out + beta * np.asarray(C_in, dtype=np.float64)
    return out


# --- sampled output tiles, for operands too large to rebuild whole ----------

def _op_row_panel(t: TLRTiles, op: str, r0: int, r1: int) -> np.ndarray:
    """Rows [r0, r1) of op(stored) as a dense float64 array."""
    if op == "N":
        sizes, other = t.row_sizes, t.col_sizes
    else:
        sizes, other = t.col_sizes, t.row_sizes
    off = offsets(sizes)
    total = sum(other)
    out = np.zeros((r1 - r0, total))
    oo = offsets(other)
    for a, s in enumerate(sizes):
        lo, hi = max(r0, off[a]), min(r1, off[a] + s)
        if lo >= hi:
            continue
        for c, w in enumerate(other):
            tile = dense_tile(t, a, c) if op == "N" else dense_tile(t, c, a).T
            out[lo - r0:hi - r0, oo[c]:oo[c] + w] = tile[lo - off[a]:hi - off[a], :]
    return out


def _op_col_panel(t: TLRTiles, op: str, c0: int, c1: int) -> np.ndarray:
    """Columns [c0, c1) of op(stored) as a dense float64 array."""
    return _op_row_panel(t, "T" if op == "N" else "N", c0, c1).T


def gemm_reference_block(alpha: float, opA: str, A: TLRTiles, opB: str, B,
                         beta: float, C_block: Optional[np.ndarray],
                         rows: Tuple[int, int], cols: Tuple[int, int],
                         timings: Optional[dict] = None) -> np.ndarray:
    """Block C[rows[0]:rows[1], cols[0]:cols[1]] of the same product, built from
    the row panel of op(A) and the column panel of op(B) only.  ``timings``, if
    given, accumulates the seconds spent rebuilding the panels
    ("reconstruct_s") and multiplying ("matmul_s")."""
    t0 = time.perf_counter()
    if isinstance(A, TLRTiles):
        Ap = _op_row_panel(A, opA, rows[0], rows[1])
    else:
        Ad = np.asarray(A)
        Ap = (Ad[rows[0]:rows[1], :] if opA == "N" else Ad[:, rows[0]:rows[1]].T).astype(np.float64)
    if isinstance(B, TLRTiles):
        Bp = _op_col_panel(B, opB, cols[0], cols[1])
    else:
        Bd = np.asarray(B)
        Bp = (Bd[:, cols[0]:cols[1]] if opB == "N" else Bd[cols[0]:cols[1], :].T).astype(np.float64)
    t1 = time.perf_counter()
    out = alpha * (Ap @ Bp)
    if beta != 0.0:
        out = out + beta * np.asarray(C_block, dtype=np.float64)
    if timings is not None:
        timings["reconstruct_s"] = timings.get("reconstruct_s", 0.0) + (t1 - t0)
        timings["matmul_s"] = timings.get("matmul_s", 0.0) + (time.perf_counter() - t1)
    return out


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_F / ||ref||_F in float64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)

"""The per-contraction-tile loop, in plain Python scalar loops (tiny grids only).

Follows "Tile-Low-Rank GEMM: Designing Storage Around the Contraction",
section "Many small GEMMs": for each contraction tile k and every output tile
pair (i, j), form the coupling S = V_ik^T W_kj, the right product
T = S Z_kj^T, and add U_ik T into C_ij.  Terms that meet a dense diagonal tile
use that tile in place of the factor pair, as "TLR Matrix Multiplication"
splits A = D_A + O_A and B = D_B + O_B (section "Regular TLR GEMM", the D_A D_B,
O_A D_B, D_A O_B and O_A O_B products).

No BLAS is used: every product is an explicit triple loop, and the loop counts
the multiply-adds it performs (2 flops each).  With ``assoc='left'`` the
low-rank terms are evaluated as (U_ik S) Z_kj^T and the O_A D_B terms as
U (V^T D); this is the order "Association order and workspace" describes.  The
flop count of the loop is therefore an independent count of the useful work of
either association order.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from tlr_inputs import TLRTiles

Mat = List[List[float]]


class _Counter:
    def __init__(self):
        self.flops = 0


def _mat(a) -> Mat:
    a = np.asarray(a, dtype=np.float64)
    return [[float(a[r, c]) for c in range(a.shape[1])] for r in range(a.shape[0])]


def _t(a: Mat, ncols_if_empty: int = 0) -> Mat:
    if not a:
        return [[] for _ in range(ncols_if_empty)]
    return [[a[r][c] for r in range(len(a))] for c in range(len(a[0]))]


def _mm(x: Mat, y: Mat, m: int, k: int, n: int, cnt: _Counter) -> Mat:
    """(m x k) times (k x n) with explicit loops."""
    out = [[0.0] * n for _ in range(m)]
    for r in range(m):
        for c in range(n):
            acc = 0.0
            for t in range(k):
                acc += x[r][t] * y[t][c]
            out[r][c] = acc
    cnt.flops += 2 * m * n * k
    return out


def _op_tile(t: TLRTiles, op: str, i: int, k: int):
    """Tile (i, k) of op(stored) as ('D', dense) or ('LR', outer, inner, r).

    For op = T the tile is the transpose of stored tile (k, i): its outer
    factor is the stored inner factor and vice versa ("Where fusion stops",
    Transposes)."""
    a, c = (i, k) if op == "N" else (k, i)
    if t.has_diag and a == c:
        d = _mat(t.diag[a])
        return ("D", d if op == "N" else _t(d))
    r = int(t.ranks[a, c])
    rs, cs = t.row_sizes, t.col_sizes
    if r == 0:
        s_out = rs[a] if op == "N" else cs[c]
        s_in = cs[c] if op == "N" else rs[a]
        return ("LR", [[] for _ in range(s_out)], [[] for _ in range(s_in)], 0)
    u, v = _mat(t.U[(a, c)]), _mat(t.V[(a, c)])
    return ("LR", u, v, r) if op == "N" else ("LR", v, u, r)


def tile_loop(alpha: float, opA: str, A: TLRTiles, opB: str, B, beta: float,
              C_in: Optional[np.ndarray], assoc: str = "right") -> Tuple[np.ndarray, int]:
    """C = alpha op(A) op(B) + beta C_in by the per-k tile loop.

    Returns (C as float64 array, flops performed).  ``B`` may be a dense array;
    then each op(B) tile is dense and a low-rank A tile is applied as
    U (V^T B_kj).  ``A`` may be a dense array (with a TLR ``B``): its row panel
    k-block is one dense tile per contraction tile (the contraction tiles are
    op(B)'s row tiles) and a low-rank B tile is applied as (A_k W_kj) Z_kj^T.
    C_in is not read when beta == 0."""
    if assoc not in ("right", "left"):
        raise ValueError(assoc)
    cnt = _Counter()
    dense_A = not isinstance(A, TLRTiles)
    if dense_A:
        Ad = np.asarray(A, dtype=np.float64)
        Ad = Ad if opA == "N" else Ad.T
        mrows = [Ad.shape[0]] if Ad.shape[0] > 0 else []
        ksz = B.row_sizes if opB == "N" else B.col_sizes
        from .reference import offsets as _off
        kao = _off(ksz)
    elif opA == "N":
        mrows, ksz = A.row_sizes, A.col_sizes
    else:
        mrows, ksz = A.col_sizes, A.row_sizes
    dense_B = not isinstance(B, TLRTiles)
    if dense_B:
        Bd = np.asarray(B, dtype=np.float64)
        Bd = Bd if opB == "N" else Bd.T
        from .reference import offsets as _off
        ncols_total = Bd.shape[1]
        ncols = [ncols_total] if ncols_total > 0 else []
        kro = _off(ksz)
    else:
        ncols = B.col_sizes if opB == "N" else B.row_sizes
    qm, qk, qn = len(mrows), len(ksz), len(ncols)
    # C <- beta C  (beta == 0: C is not read)
    C = [[[[0.0] * ncols[j] for _ in range(mrows[i])] for j in range(qn)] for i in range(qm)]
    if beta != 0.0:
        from .reference import offsets as _off
        ro, co = _off(mrows), _off(ncols)
        Cin = np.asarray(C_in, dtype=np.float64)
        for i in range(qm):
            for j in range(qn):
                for r in range(mrows[i]):
                    for c in range(ncols[j]):
                        C[i][j][r][c] = beta * float(Cin[ro[i] + r, co[j] + c])
    for k in range(qk):
        for i in range(qm):
            ta = ("D", _mat(Ad[:, kao[k]:kao[k] + ksz[k]])) if dense_A else _op_tile(A, opA, i, k)
            for j in range(qn):
                si, sk, sj = mrows[i], ksz[k], ncols[j]
                if dense_B:
                    tb = ("D", _mat(Bd[kro[k]:kro[k] + sk, :]))
                else:
                    tb = _op_tile(B, opB, k, j)
                if ta[0] == "D" and tb[0] == "D":
                    upd = _mm(ta[1], tb[1], si, sk, sj, cnt)
                elif ta[0] == "D":            # D_A (W Z^T), evaluated (D W) Z^T
                    _, w, z, rb = tb
                    if rb == 0:
                        continue
                    x = _mm(ta[1], w, si, sk, rb, cnt)
                    upd = _mm(x, _t(z, rb), si, rb, sj, cnt)
                elif tb[0] == "D":            # (U V^T) D_B
                    _, u, v, ra = ta
                    if ra == 0:
                        continue
                    vtd = _mm(_t(v, ra), tb[1], ra, sk, sj, cnt)
                    upd = _mm(u, vtd, si, ra, sj, cnt)
                else:                          # U (V^T W) Z^T
                    _, u, v, ra = ta
                    _, w, z, rb = tb
                    if ra == 0 or rb == 0:
                        continue
                    s = _mm(_t(v, ra), w, ra, sk, rb, cnt)          # coupling
                    if assoc == "right":
                        tt = _mm(s, _t(z, rb), ra, rb, sj, cnt)     # right product
                        upd = _mm(u, tt, si, ra, sj, cnt)           # update
                    else:
                        y = _mm(u, s, si, ra, rb, cnt)
                        upd = _mm(y, _t(z, rb), si, rb, sj, cnt)
                ci = C[i][j]
                for r in range(si):
                    row, urow = ci[r], upd[r]
                    for c in range(sj):
                        row[c] += alpha * urow[c]
    from .reference import offsets as _off
    ro, co = _off(mrows), _off(ncols)
    out = np.zeros((sum(mrows), sum(ncols)))
    for i in range(qm):
        for j in range(qn):
            if mrows[i] and ncols[j]:
                out[ro[i]:ro[i] + mrows[i], co[j]:co[j] + ncols[j]] = np.array(C[i][j])
    return out, cnt.flops

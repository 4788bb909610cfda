"""TLR-output product and dense-to-TLR compression, in float64 on the CPU.

"TLR Matrix Multiplication", section "Introduction: TLR GEMM": each of A, B
and C may be stored densely or in TLR format, with dense diagonal tiles and
every off-diagonal tile a factor pair of its own rank; the TLR-output cases
extend the dense-output product.  The pages give no algorithm and no
accuracy target for them.  Reading used here (the plainest one):

  1. the result tile is the exact one, X_ij = alpha (op(A) op(B))_ij +
     beta C_ij, with C rebuilt from its own factors (C read only when
     beta != 0);
  2. a diagonal tile stays dense: C_ii <- X_ii;
  3. an off-diagonal tile is replaced by the truncated singular value
     decomposition of X_ij of the smallest rank r whose discarded part meets
     the tolerance tol relative to the tile:
         sqrt(sum_{k >= r} sigma_k^2) <= tol * ||X_ij||_F
     (sigma_0 >= sigma_1 >= ... the singular values of X_ij).  By the
     Eckart-Young theorem no factorisation of smaller rank meets tol, and
     the rank-r truncation's error is exactly that tail.  The factors are
     U_ij = left singular vectors times sigma, V_ij = right singular vectors
     (any factor pair with the same product is an equally valid result).

TEST INFRASTRUCTURE ONLY, like the rest of this package.  It uses numpy's SVD
as a library step.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from tlr_inputs import TLRTiles, tile_sizes

from .reference import gemm_reference, offsets, reconstruct


def truncation_rank(sigma: np.ndarray, fro: float, tol: float) -> int:
    """Smallest r with sqrt(sum_{k >= r} sigma_k^2) <= tol * fro (sigma sorted
    in decreasing order)."""
    s = np.asarray(sigma, dtype=np.float64)
    limit = (tol * fro) ** 2
    tail = 0.0
    r = len(s)
    # walk from the smallest singular value up while the tail stays within the limit
    for k in range(len(s) - 1, -1, -1):
        if tail + s[k] * s[k] <= limit:
            tail += s[k] * s[k]
            r = k
        else:
            break
    return r


def truncate_tile(X: np.ndarray, tol: float) -> Tuple[np.ndarray, np.ndarray, int, np.ndarray]:
    """(U, V, r, sigma): the truncated SVD of one tile, U = left vectors times
    sigma (s_i x r), V = right vectors (s_j x r)."""
    X = np.asarray(X, dtype=np.float64)
    if X.size == 0:
        return np.zeros((X.shape[0], 0)), np.zeros((X.shape[1], 0)), 0, np.zeros(0)
    Us, s, Vt = np.linalg.svd(X, full_matrices=False)
    r = truncation_rank(s, float(np.linalg.norm(X)), tol)
    return Us[:, :r] * s[:r], Vt[:r, :].T.copy(), r, s


def compress(X: np.ndarray, b: int, has_diag: bool, tol: float) -> TLRTiles:
    """A dense matrix as a TLR operand: tile grid of size b, the diagonal
    tiles dense (square matrices only), every other tile truncated as above."""
    X = np.asarray(X, dtype=np.float64)
    rows, cols = X.shape
    rs, cs = tile_sizes(rows, b), tile_sizes(cols, b)
    ro, co = offsets(rs), offsets(cs)
    R = np.zeros((len(rs), len(cs)), dtype=np.int32)
    U: Dict[Tuple[int, int], np.ndarray] = {}
    V: Dict[Tuple[int, int], np.ndarray] = {}
    D: Optional[List[np.ndarray]] = [] if has_diag else None
    for i in range(len(rs)):
        for j in range(len(cs)):
            tile = X[ro[i]:ro[i] + rs[i], co[j]:co[j] + cs[j]]
            if has_diag and i == j:
                D.append(tile.copy())
                continue
            u, v, r, _ = truncate_tile(tile, tol)
            R[i, j] = r
            U[(i, j)], V[(i, j)] = u, v
    return TLRTiles(rows, cols, b, R, D, U, V, "f64")


def tlr_output_reference(alpha: float, opA: str, A, opB: str, B, beta: float, C: Optional[TLRTiles],
                         tol: float) -> TLRTiles:
    """C <- alpha op(A) op(B) + beta C with C in TLR format: the exact product
    (C rebuilt from its factors, read only when beta != 0), then every
    off-diagonal tile truncated to tol.  The output keeps C's tile size and
    its dense diagonal."""
    C_in = None if beta == 0.0 else reconstruct(C)
    X = gemm_reference(alpha, opA, A, opB, B, beta, C_in)
    return compress(X, C.b, C.has_diag, tol)


def tile_errors(T: TLRTiles, X: np.ndarray) -> np.ndarray:
    """Per off-diagonal tile ||U V^T - X_ij||_F / ||X_ij||_F (0 where X_ij = 0
    and the tile is empty); NaN on the diagonal."""
    rs, cs = T.row_sizes, T.col_sizes
    ro, co = offsets(rs), offsets(cs)
    out = np.full((len(rs), len(cs)), np.nan)
    for i in range(len(rs)):
        for j in range(len(cs)):
            if T.has_diag and i == j:
                continue
            x = np.asarray(X[ro[i]:ro[i] + rs[i], co[j]:co[j] + cs[j]], dtype=np.float64)
            u = np.asarray(T.U[(i, j)], dtype=np.float64)
            v = np.asarray(T.V[(i, j)], dtype=np.float64)
            d = np.linalg.norm(u @ v.T - x)
            n = np.linalg.norm(x)
            out[i, j] = d / n if n > 0 else d
    return out

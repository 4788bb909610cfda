"""Rank-metadata arithmetic of the three-stage TLR product (integers only).

Follows "Tile-Low-Rank GEMM: Designing Storage Around the Contraction":
  * "Packing for the contraction": rho_i is the rank sum of tile row i of the
    outer factors, p_i(k) the prefix sum that locates tile k in it.
  * "One product, three stages": Stage 1 is one coupling GEMM per contraction
    tile k of shape (sum_i r_ik, sum_j r_kj, n_k); Stage 2 is one task per
    (i, k, j) of shape (r_ik, n_j, r_kj) writing row block k / column block j
    of the terminal matrix T_i; Stage 3 is one GEMM per tile row of shape
    (m_i, sum_j n_j, rho_i).
  * "Association order and workspace": the left order ends with one GEMM per
    tile column, (sum_i m_i, n_j, gamma_j) with gamma_j = sum_k r_kj; the
    final-stage costs are F_R = 2 sum_i m_i rho_i sum_j n_j and
    F_L = 2 sum_j n_j gamma_j sum_i m_i.
Dense diagonal tiles follow "TLR Matrix Multiplication" ("Regular TLR GEMM":
A = D_A + O_A, B = D_B + O_B).

Here ``RA`` and ``RB`` are the rank tables of op(A) and op(B) (already
transposed when op = T), ``ms``/``ks``/``ns`` the tile sizes along the rows of
C, the contraction, and the columns of C, and ``dA``/``dB`` say whether op(A)
/ op(B) has dense diagonal tiles.  Every function loops over tiles plainly.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def op_ranks(R: np.ndarray, op: str) -> np.ndarray:
    return np.asarray(R) if op == "N" else np.asarray(R).T


def rho(RA) -> List[int]:
    """Row rank sums of op(A): rho_i = sum_k r_ik."""
    RA = np.asarray(RA)
    return [int(sum(int(RA[i, k]) for k in range(RA.shape[1]))) for i in range(RA.shape[0])]


def gamma(RB) -> List[int]:
    """Column rank sums of op(B): gamma_j = sum_k r_kj."""
    RB = np.asarray(RB)
    return [int(sum(int(RB[k, j]) for k in range(RB.shape[0]))) for j in range(RB.shape[1])]


def stage1_shapes(RA, RB, ks, I=None, J=None) -> List[Tuple[int, int, int]]:
    """(M, N, K) of the coupling GEMM of each contraction tile k."""
    RA, RB = np.asarray(RA), np.asarray(RB)
    I = range(RA.shape[0]) if I is None else I
    J = range(RB.shape[1]) if J is None else J
    out = []
    for k in range(RA.shape[1]):
        M = sum(int(RA[i, k]) for i in I)
        N = sum(int(RB[k, j]) for j in J)
        out.append((M, N, ks[k]))
    return out


def stage3_shapes(RA, RB, ms, ns, order: str, I=None, J=None) -> List[Tuple[int, int, int]]:
    """(M, N, K) of the final GEMMs: one per tile row (right) or column (left)."""
    RA, RB = np.asarray(RA), np.asarray(RB)
    I = list(range(RA.shape[0])) if I is None else list(I)
    J = list(range(RB.shape[1])) if J is None else list(J)
    if order == "right":
        r = rho(RA)
        width = sum(ns[j] for j in J)
        return [(ms[i], width, r[i]) for i in I]
    g = gamma(RB)
    height = sum(ms[i] for i in I)
    return [(height, ns[j], g[j]) for j in J]


def final_stage_flops(RA, RB, ms, ns, order: str) -> int:
    """F_R or F_L of the whole product."""
    return sum(2 * M * N * K for (M, N, K) in stage3_shapes(RA, RB, ms, ns, order))


def coupling_products(RA, RB, ks) -> List[Tuple[int, int, int, Tuple[int, int, int]]]:
    """Every tile-level coupling product (i, k, j, (r_ik, r_kj, n_k)) with both
    ranks non-zero."""
    RA, RB = np.asarray(RA), np.asarray(RB)
    out = []
    for i in range(RA.shape[0]):
        for k in range(RA.shape[1]):
            for j in range(RB.shape[1]):
                if RA[i, k] > 0 and RB[k, j] > 0:
                    out.append((i, k, j, (int(RA[i, k]), int(RB[k, j]), ks[k])))
    return out


def stage2_tasks(RA, RB, ms, ns, order: str):
    """Tile-level Stage-2 tasks: right (r_ik, n_j, r_kj) written into T_i,
    left (m_i, r_kj, r_ik) written into Y_j."""
    RA, RB = np.asarray(RA), np.asarray(RB)
    out = []
    for i in range(RA.shape[0]):
        for k in range(RA.shape[1]):
            for j in range(RB.shape[1]):
                if RA[i, k] > 0 and RB[k, j] > 0:
                    if order == "right":
                        out.append((int(RA[i, k]), ns[j], int(RB[k, j])))
                    else:
                        out.append((ms[i], int(RB[k, j]), int(RA[i, k])))
    return out


def terminal_workspace(RA, RB, ms, ns, order: str) -> Tuple[int, int]:
    """Shape of the stacked terminal matrices: right (sum_i rho_i, sum_j n_j),
    left (sum_i m_i, sum_j gamma_j)."""
    if order == "right":
        return (sum(rho(RA)), sum(ns))
    return (sum(ms), sum(gamma(RB)))


def useful_flops(RA, RB, ms, ks, ns, dA: bool, dB: bool, order: str,
                 I: Optional[Sequence[int]] = None, J: Optional[Sequence[int]] = None) -> int:
    """Useful flops of one rectangle of output tiles (whole C by default),
    counted term by term over (i, k, j):

      D_A D_B  (i = k = j)          2 m_i^3
      D_A O_B  (k = i)              (D W) then times Z^T
      O_A D_B  (k = j)              (V^T D) then U times it
      O_A O_B                       coupling + right product + update (right)
                                    coupling + U S + times Z^T (left)
    The coupling S_ikj is shared by every rectangle row/column only within a
    rectangle; here it is counted once per (i, k, j) like the tile loop."""
    RA, RB = np.asarray(RA), np.asarray(RB)
    I = range(RA.shape[0]) if I is None else I
    J = range(RB.shape[1]) if J is None else J
    F = 0
    for i in I:
        for k in range(RA.shape[1]):
            for j in J:
                mi, sk, nj = ms[i], ks[k], ns[j]
                a_d = dA and i == k
                b_d = dB and k == j
                if a_d and b_d:
                    F += 2 * mi * sk * nj
                elif a_d:
                    rb = int(RB[k, j])
                    F += 2 * mi * sk * rb + 2 * mi * rb * nj
                elif b_d:
                    ra = int(RA[i, k])
                    F += 2 * ra * sk * nj + 2 * mi * ra * nj
                else:
                    ra, rb = int(RA[i, k]), int(RB[k, j])
                    if ra == 0 or rb == 0:
                        continue
                    F += 2 * ra * rb * sk
                    if order == "right":
                        F += 2 * ra * rb * nj + 2 * mi * ra * nj
                    else:
                        F += 2 * mi * ra * rb + 2 * mi * rb * nj
    return F


def useful_flops_dense_b(RA, ms, ks, ncols: int, dA: bool, I=None) -> int:
    """Useful flops of op(A) (TLR) times a dense op(B) with ``ncols`` columns:
    per (i, k) either D_ii B_k (k = i) or U_ik (V_ik^T B_k)."""
    RA = np.asarray(RA)
    I = range(RA.shape[0]) if I is None else I
    F = 0
    for i in I:
        for k in range(RA.shape[1]):
            if dA and i == k:
                F += 2 * ms[i] * ks[k] * ncols
            else:
                ra = int(RA[i, k])
                F += 2 * ra * ks[k] * ncols + 2 * ms[i] * ra * ncols
    return F


def useful_flops_dense_a(RB, ks, ns, mrows: int, dB: bool, J=None) -> int:
    """Useful flops of a dense op(A) with ``mrows`` rows times op(B) (TLR): per
    (k, j) either A_k D_kk (k = j) or (A_k W_kj) Z_kj^T."""
    RB = np.asarray(RB)
    J = range(RB.shape[1]) if J is None else J
    F = 0
    for k in range(RB.shape[0]):
        for j in J:
            if dB and k == j:
                F += 2 * mrows * ks[k] * ns[j]
            else:
                rb = int(RB[k, j])
                F += 2 * mrows * ks[k] * rb + 2 * mrows * rb * ns[j]
    return F


def workspace_elements(RA, RB, ms, ks, ns, dA: bool, dB: bool, order: str,
                       I: Sequence[int], J: Sequence[int]) -> Dict[str, int]:
    """Element counts of the intermediates one rectangle needs:
    S (every coupling block S_k), the terminal matrices (T_i for right, Y_j for
    left) and the diagonal-term products (D_A W for right, V^T D_B for left)."""
    RA, RB = np.asarray(RA), np.asarray(RB)
    I, J = list(I), list(J)
    S = 0
    for k in range(RA.shape[1]):
        S += sum(int(RA[i, k]) for i in I) * sum(int(RB[k, j]) for j in J)
    if order == "right":
        r = rho(RA)
        width = sum(ns[j] for j in J)
        term = sum(r[i] * width for i in I)
        x = sum(ms[i] * sum(int(RB[i, j]) for j in J) for i in I) if dA else 0
    else:
        g = gamma(RB)
        height = sum(ms[i] for i in I)
        term = sum(height * g[j] for j in J)
        x = sum(sum(int(RA[i, j]) for i in I) * ns[j] for j in J) if dB else 0
    return {"S": S, "terminal": term, "diag": x}

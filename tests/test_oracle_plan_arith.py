"""Rank-metadata arithmetic of the oracle, pinned to the pages and to brute force.

* The worked example of "Tile-Low-Rank GEMM: Designing Storage Around the
  Contraction" (sections "One product, three stages", "Association order and
  workspace"): printed Stage-1 and Stage-3 GEMM shapes, rho, gamma, the
  final-stage costs 2b^2*528 and 2b^2*608, the terminal workspace sizes and
  the count of coupling products and shapes (fixture tests/golden/
  worked_example.json, both completions of the lost rank table).
* A closed form: for uniform ranks r_A, r_B on a q x q grid of b x b tiles
  with dense diagonals, F_R - F_L = 2 b^2 q (q-1)^2 (r_A - r_B), so the right
  order is cheaper iff r_A < r_B ("TLR Matrix Multiplication", the O_A O_B
  terms: order by min(r_A, r_B)).
* The flop count of the brute-force tile loop (which counts the multiply-adds
  it performs) equals the oracle's useful-flop count, per association order,
  on random tiny grids with and without diagonals and with a dense B.
"""
import json
import os

import numpy as np
import pytest

from oracle import brute, plan_arith as pa
from tlr_inputs import random_tlr, tile_sizes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


@pytest.mark.parametrize("cand", sorted(GOLD["B_ranks_candidates"]))
def test_worked_example(cand):
    b = GOLD["b"]
    RA = np.array(GOLD["A_ranks"])
    RB = np.array(GOLD["B_ranks_candidates"][cand])
    P = GOLD["printed"]
    ms, ks, ns = [b, b], [b, b, b], [b, b, b]
    assert [list(s) for s in pa.stage1_shapes(RA, RB, ks)] == P["stage1_shapes_MNK"]
    assert [list(s) for s in pa.stage3_shapes(RA, RB, ms, ns, "right")] == P["stage3_right_shapes_MNK"]
    assert pa.rho(RA) == P["rho"]
    assert pa.gamma(RB) == P["gamma"]
    FR = pa.final_stage_flops(RA, RB, ms, ns, "right")
    FL = pa.final_stage_flops(RA, RB, ms, ns, "left")
    assert FR == 2 * b * b * P["F_R_over_2b2"]
    assert FL == 2 * b * b * P["F_L_over_2b2"]
    assert (FR < FL) == (P["chosen_order"] == "right")
    assert abs(1 - FR / FL - 0.13) < 0.01          # right does about 13 % less
    assert list(pa.terminal_workspace(RA, RB, ms, ns, "right")) == P["terminal_right_shape"]
    assert list(pa.terminal_workspace(RA, RB, ms, ns, "left")) == P["terminal_left_shape"]
    assert [pa.rho(RA)[0], sum(ns)] == P["T_1_shape"]
    cp = pa.coupling_products(RA, RB, ks)
    assert len(cp) == P["coupling_products"]
    assert len({c[3] for c in cp}) == P["coupling_distinct_shapes"]
    k1 = [c for c in cp if c[1] == 0]
    assert len(k1) == P["k1_products"] and len({c[3] for c in k1}) == P["k1_distinct_shapes"]
    t2 = pa.stage2_tasks(RA, RB, ms, ns, "right")
    assert len(t2) == P["stage2_tasks"] and len(set(t2)) == P["stage2_distinct_shapes"]
    # Stage 2 costs the same in both orders for square tiles
    s2r = sum(2 * a * c * d for (a, c, d) in t2)
    s2l = sum(2 * a * c * d for (a, c, d) in pa.stage2_tasks(RA, RB, ms, ns, "left"))
    assert s2r == s2l


@pytest.mark.parametrize("q,b,ra,rb", [(3, 8, 2, 5), (4, 6, 4, 1), (5, 4, 2, 2), (2, 9, 7, 3)])
def test_uniform_rank_closed_form(q, b, ra, rb):
    n = q * b
    RA = np.full((q, q), ra)
    np.fill_diagonal(RA, 0)
    RB = np.full((q, q), rb)
    np.fill_diagonal(RB, 0)
    s = [b] * q
    FR = pa.useful_flops(RA, RB, s, s, s, True, True, "right")
    FL = pa.useful_flops(RA, RB, s, s, s, True, True, "left")
    assert FR - FL == 2 * b * b * q * (q - 1) ** 2 * (ra - rb)
    # every term of the right order, summed by hand
    by_hand = (2 * q * b ** 3                      # D_A D_B
               + 2 * q * (q - 1) * ra * b * b      # V^T D_B
               + 2 * q * (q - 1) * b * b * rb      # D_A W
               + 2 * q * (q - 1) * b * rb * b      # (D_A W) Z^T
               + q * 2 * ((q - 1) * ra) * ((q - 1) * rb) * b   # coupling
               + 2 * q * (q - 1) ** 2 * ra * rb * b            # right product
               + 2 * q * b * ((q - 1) * ra) * n)               # update
    assert FR == by_hand


def _rand(seed, n, b, diag, dense_b=False):
    rng = np.random.default_rng(seed)
    A = random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
    B = rng.standard_normal((n, n)) if dense_b else random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
    return A, B


@pytest.mark.parametrize("seed,n,b,diag", [(1, 9, 3, True), (2, 10, 4, True), (3, 7, 2, False),
                                           (4, 11, 4, False), (5, 5, 5, True)])
@pytest.mark.parametrize("opA,opB", [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")])
def test_brute_force_flops_equal_useful_flops(seed, n, b, diag, opA, opB):
    A, B = _rand(seed, n, b, diag)
    RA, RB = pa.op_ranks(A.ranks, opA), pa.op_ranks(B.ranks, opB)
    s = tile_sizes(n, b)
    for order in ("right", "left"):
        _, flops = brute.tile_loop(1.0, opA, A, opB, B, 0.0, None, order)
        assert flops == pa.useful_flops(RA, RB, s, s, s, diag, diag, order)


@pytest.mark.parametrize("seed,n,b", [(6, 9, 3), (7, 10, 4), (8, 4, 4)])
@pytest.mark.parametrize("opA", ["N", "T"])
def test_brute_force_flops_dense_b(seed, n, b, opA):
    A, Bd = _rand(seed, n, b, True, dense_b=True)
    RA = pa.op_ranks(A.ranks, opA)
    s = tile_sizes(n, b)
    _, flops = brute.tile_loop(1.0, opA, A, "N", Bd, 0.0, None, "right")
    assert flops == pa.useful_flops_dense_b(RA, s, s, n, True)


def test_workspace_elements_worked_example():
    b = GOLD["b"]
    RA = np.array(GOLD["A_ranks"])
    RB = np.array(GOLD["B_ranks_candidates"]["B_a"])
    ms, ks, ns = [b, b], [b, b, b], [b, b, b]
    w = pa.workspace_elements(RA, RB, ms, ks, ns, False, False, "right", [0, 1], [0, 1, 2])
    assert w["terminal"] == 176 * 768 and w["diag"] == 0
    assert w["S"] == sum(M * N for (M, N, K) in GOLD["printed"]["stage1_shapes_MNK"])
    w = pa.workspace_elements(RA, RB, ms, ks, ns, False, False, "left", [0, 1], [0, 1, 2])
    assert w["terminal"] == 512 * 304


# Hand counts of one rectangle's intermediates, with dense diagonals and
# sub-rectangles ("TLR Matrix Multiplication", "The easy terms": the diagonal
# term of A gives X_i = D_A,ii W_{i,J}, s_i rows by sum_{j in J} r^B_ij
# columns; that of B gives X'_j = V_{I,j}^T D_B,jj, sum_{i in I} r^A_ij rows
# by s_j columns; "Tile-Low-Rank GEMM: Designing Storage Around the
# Contraction", "One product, three stages": S_k is sum_{i in I} r_ik by
# sum_{j in J} r_kj, T_i is rho_i by the width of J, Y_j the height of I by
# gamma_j).  Tile sizes differ along the three dimensions, so a swapped size
# list changes the count.  Every number below was added up by hand.
#
# Case R: op(A) 11 x 11 with a dense diagonal (tiles 4, 4, 3), op(B) 11 x 14
# without one (column tiles 4, 4, 4, 2); I = tile rows {1, 2}, J = tile
# columns {1, 2, 3}.
#   S: k=0 (3+2)(2+0+3)=25, k=1 (0+2)(0+2+1)=6, k=2 (1+0)(1+1+0)=2 -> 33
#   right: rho_1 = 4, rho_2 = 4, width 4+4+2 = 10 -> T 80;
#          X_1 = 4 rows x (0+2+1) = 12, X_2 = 3 rows x (1+1+0) = 6 -> 18
#   left:  gamma = 3, 3, 4, height 4+3 = 7 -> Y 70; no diagonal in B -> 0
# Case L: op(A) 14 x 11 without a diagonal (row tiles 4, 4, 4, 2), op(B)
# 11 x 11 with one (tiles 4, 4, 3); I = {0, 2, 3}, J = {0, 2}.
#   S: k=0 (1+0+1)(0+1)=2, k=1 (0+3+1)(1+3)=16, k=2 (2+1+1)(2+0)=8 -> 26
#   left:  gamma_0 = 3, gamma_2 = 4, height 4+4+2 = 10 -> Y 70;
#          X'_0 = (1+0+1) x 4 = 8, X'_2 = (2+1+1) x 3 = 12 -> 20
#   right: rho = 3, 4, 3, width 4+3 = 7 -> T 70; no diagonal in A -> 0
WS_R = dict(RA=[[0, 1, 2], [3, 0, 1], [2, 2, 0]], RB=[[1, 2, 0, 3], [1, 0, 2, 1], [2, 1, 1, 0]],
            ms=[4, 4, 3], ks=[4, 4, 3], ns=[4, 4, 4, 2], dA=True, dB=False, I=[1, 2], J=[1, 2, 3],
            right={"S": 33, "terminal": 80, "diag": 18}, left={"S": 33, "terminal": 70, "diag": 0})
WS_L = dict(RA=[[1, 0, 2], [2, 1, 0], [0, 3, 1], [1, 1, 1]], RB=[[0, 2, 1], [1, 0, 3], [2, 1, 0]],
            ms=[4, 4, 4, 2], ks=[4, 4, 3], ns=[4, 4, 3], dA=False, dB=True, I=[0, 2, 3], J=[0, 2],
            right={"S": 26, "terminal": 70, "diag": 0}, left={"S": 26, "terminal": 70, "diag": 20})


@pytest.mark.parametrize("case", [WS_R, WS_L], ids=["diag_A", "diag_B"])
@pytest.mark.parametrize("order", ["right", "left"])
def test_workspace_elements_hand_counts(case, order):
    w = pa.workspace_elements(np.array(case["RA"]), np.array(case["RB"]), case["ms"], case["ks"], case["ns"],
                              case["dA"], case["dB"], order, case["I"], case["J"])
    assert w == case[order]

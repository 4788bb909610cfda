"""Dense A times a TLR B (dense C): the oracle pinned for that operand pair.

"Tile-Low-Rank GEMM: Designing Storage Around the Contraction" covers
C <- alpha op(A) op(B) + beta C with a dense C and one or both operands TLR
(introduction).  With A dense, each contraction tile k of op(A) is a dense
panel; the pins:

* the definition (oracle.reference: rebuild op(B), one BLAS product) equals
  the per-k tile loop (oracle.brute, scalar loops, (A_k W_kj) Z_kj^T for a
  low-rank tile and A_k D_kk for a dense diagonal one) to 1e-13, over tile
  grids with ragged last tiles, all op pairs, beta in {0 (C all NaN), 0.5},
  rectangular A and B with and without dense diagonals;
* the loop's own multiply-add count equals the rank arithmetic of
  oracle.plan_arith.useful_flops_dense_a, term by term;
* (op(A) op(B))^T = op(B)^T op(A)^T: the dense-A definition equals the
  transpose of the TLR x dense one with the ops flipped;
* closed forms: every off-diagonal rank 0 leaves C[:, j] = A[:, j-block] D_jj
  (block columns times the diagonal tiles); B = identity tiles
  (D_jj = I, ranks 0) gives alpha A + beta C.
"""
import itertools

import numpy as np
import pytest

from oracle import brute, plan_arith as pa, reference
from tlr_inputs import random_tlr

FLIP = {"N": "T", "T": "N"}


def _dense_a(rng, m, k, opA):
    return rng.standard_normal((m, k) if opA == "N" else (k, m))


GRID = [(q, b, rem) for q in (1, 2, 3) for b in (2, 3, 5) for rem in (0, 1) if rem < b]


@pytest.mark.parametrize("q,b,rem", GRID)
def test_definition_equals_tile_loop(q, b, rem):
    n = q * b if rem == 0 else (q - 1) * b + rem
    for t, (opA, opB, beta, diag) in enumerate(itertools.product("NT", "NT", (0.0, 0.5), (True, False))):
        rng = np.random.default_rng(1000 * q + 100 * b + 10 * rem + t)
        m = n + 3 - (t % 5)                  # rows of C independent of the grid
        B = random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
        A = _dense_a(rng, m, n, opA)
        C = np.full((m, n), np.nan) if beta == 0.0 else rng.standard_normal((m, n))
        ref = reference.gemm_reference(0.75, opA, A, opB, B, beta, C)
        bf, flops = brute.tile_loop(0.75, opA, A, opB, B, beta, C)
        assert np.all(np.isfinite(ref))
        assert reference.rel_fro(bf, ref) <= 1e-13, (q, b, rem, opA, opB, beta, diag)
        RB = pa.op_ranks(B.ranks, opB)
        ks = B.row_sizes if opB == "N" else B.col_sizes
        ns = B.col_sizes if opB == "N" else B.row_sizes
        assert flops == pa.useful_flops_dense_a(RB, ks, ns, m, diag), (q, b, rem, opA, opB, diag)


def test_rectangular_b_without_diagonal():
    rng = np.random.default_rng(3)
    B = random_tlr(rng, 12, 8, 4, rank_lo=0, has_diag=False, scale=1.0)      # 3 x 2 tiles
    for opA, opB in itertools.product("NT", "NT"):
        k = 12 if opB == "N" else 8
        A = _dense_a(rng, 5, k, opA)
        ref = reference.gemm_reference(1.0, opA, A, opB, B, 0.0, None)
        bf, _ = brute.tile_loop(1.0, opA, A, opB, B, 0.0, None)
        assert reference.rel_fro(bf, ref) <= 1e-13


def test_transpose_identity():
    rng = np.random.default_rng(11)
    B = random_tlr(rng, 10, 10, 4, rank_lo=1, has_diag=True, scale=1.0)
    for opA, opB in itertools.product("NT", "NT"):
        A = _dense_a(rng, 7, 10, opA)
        got = reference.gemm_reference(1.0, opA, A, opB, B, 0.0, None)
        # op(A) op(B) = (op(B)^T op(A)^T)^T, the second a TLR x dense product
        other = reference.gemm_reference(1.0, FLIP[opB], B, FLIP[opA], A, 0.0, None)
        assert reference.rel_fro(got, other.T) <= 1e-14


def test_rank_zero_is_block_columns_times_diagonal():
    rng = np.random.default_rng(12)
    n, b = 11, 4
    B = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=0, has_diag=True, scale=1.0)
    A = rng.standard_normal((6, n))
    got, _ = brute.tile_loop(1.0, "N", A, "N", B, 0.0, None)
    off = reference.offsets(B.col_sizes)
    want = np.zeros((6, n))
    for j, s in enumerate(B.col_sizes):
        cols = slice(off[j], off[j] + s)
        D = np.asarray(B.diag[j], dtype=np.float64)
        for r in range(6):                      # scalar loops: no shared code with the reference
            for c in range(s):
                want[r, off[j] + c] = sum(A[r, off[j] + t] * D[t, c] for t in range(s))
    assert reference.rel_fro(got, want) <= 1e-14
    assert reference.rel_fro(reference.gemm_reference(1.0, "N", A, "N", B, 0.0, None), want) <= 1e-14


def test_identity_b_gives_alpha_a_plus_beta_c():
    rng = np.random.default_rng(13)
    n, b = 9, 4
    B = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=0, has_diag=True, scale=1.0)
    for j, s in enumerate(B.col_sizes):
        B.diag[j] = np.eye(s)
    A = rng.standard_normal((5, n))
    C = rng.standard_normal((5, n))
    got = reference.gemm_reference(1.5, "N", A, "N", B, -0.5, C)
    assert np.max(np.abs(got - (1.5 * A - 0.5 * C))) <= 1e-14

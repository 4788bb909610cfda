"""Invariants and textbook special cases of the dense oracle.

Each test states a fact the mathematics or the pages fix:
  * rank-0 tiles contribute nothing;
  * beta = 0 never reads C (NaN / Inf in C do not propagate);
  * storing every tile padded to r_max with zero columns gives the same C
    ("TLR Matrix Multiplication", introduction: padded vs variable storage);
  * op(A) = T equals multiplying by the explicitly transposed TLR matrix,
    built by swapping the factor families and the tile coordinates
    ("Tile-Low-Rank GEMM: Designing Storage Around the Contraction",
    "Where fusion stops", Transposes);
  * the four output regions of a matrix with boundary panels equal the 2x2
    block product of interior and boundary parts ("TLR Matrix
    Multiplication", boundary decomposition into A_int, u, v^T, gamma);
  * linearity in alpha and beta;
  * one tile (q = 1) is a plain dense GEMM; all off-diagonal ranks 0 gives a
    block-diagonal product; identity outer factors with V = A_ij^T rebuild an
    arbitrary dense matrix, so the product is the textbook one (checked
    against explicit scalar loops, not BLAS);
  * a sampled output block equals the same block of the whole product.
"""
import copy

import numpy as np
import pytest

from oracle import reference
from tlr_inputs import TLRTiles, random_tlr, tile_sizes


def _pair(seed, n=13, b=4, diag=True):
    rng = np.random.default_rng(seed)
    A = random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
    B = random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
    C = rng.standard_normal((n, n))
    return A, B, C


def test_rank_zero_tile_contributes_nothing():
    A, B, C = _pair(1)
    i, j = 0, 2
    A0 = copy.deepcopy(A)
    A0.ranks[i, j] = 0
    A0.U[(i, j)] = A0.U[(i, j)][:, :0]
    A0.V[(i, j)] = A0.V[(i, j)][:, :0]
    # zeroing the tile of the dense matrix gives the same product
    Ad = reference.reconstruct(A)
    rs = reference.offsets(A.row_sizes)
    Ad[rs[i]:rs[i] + A.row_sizes[i], rs[j]:rs[j] + A.col_sizes[j]] = 0.0
    Bd = reference.reconstruct(B)
    got = reference.gemm_reference(1.0, "N", A0, "N", B, 0.0, None)
    assert np.allclose(got, Ad @ Bd, rtol=0, atol=1e-13)


@pytest.mark.parametrize("fill", [np.nan, np.inf, -np.inf])
def test_beta_zero_ignores_c(fill):
    A, B, _ = _pair(2)
    C = np.full((13, 13), fill)
    got = reference.gemm_reference(1.3, "N", A, "T", B, 0.0, C)
    zero = reference.gemm_reference(1.3, "N", A, "T", B, 0.0, np.zeros((13, 13)))
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, zero)


def _padded(t: TLRTiles, rmax: int) -> TLRTiles:
    p = copy.deepcopy(t)
    for key in list(p.U):
        r = p.U[key].shape[1]
        p.U[key] = np.concatenate([p.U[key], np.zeros((p.U[key].shape[0], rmax - r))], axis=1)
        p.V[key] = np.concatenate([p.V[key], np.zeros((p.V[key].shape[0], rmax - r))], axis=1)
        p.ranks[key] = rmax
    return p


def test_uniform_rank_equals_padded():
    A, B, C = _pair(3, n=16, b=4)
    got = reference.gemm_reference(1.0, "N", A, "N", B, 0.5, C)
    pad = reference.gemm_reference(1.0, "N", _padded(A, 4), "N", _padded(B, 4), 0.5, C)
    assert reference.rel_fro(pad, got) <= 1e-14


def _transpose_tlr(t: TLRTiles) -> TLRTiles:
    """A^T as a TLR matrix: tile (i, k) of A^T is V_ki U_ki^T, diag D_ii^T."""
    U = {(j, i): t.V[(i, j)].copy() for (i, j) in t.U}
    V = {(j, i): t.U[(i, j)].copy() for (i, j) in t.U}
    D = None if t.diag is None else [d.T.copy() for d in t.diag]
    return TLRTiles(t.cols, t.rows, t.b, t.ranks.T.copy(), D, U, V, t.dtype)


@pytest.mark.parametrize("opA,opB", [("T", "N"), ("N", "T"), ("T", "T")])
def test_transpose_by_factor_swap(opA, opB):
    A, B, C = _pair(4, n=11, b=3)
    got = reference.gemm_reference(0.5, opA, A, opB, B, 2.0, C)
    At = _transpose_tlr(A) if opA == "T" else A
    Bt = _transpose_tlr(B) if opB == "T" else B
    exp = reference.gemm_reference(0.5, "N", At, "N", Bt, 2.0, C)
    assert reference.rel_fro(got, exp) <= 1e-14


def test_boundary_block_algebra():
    n, b = 14, 4  # m = 3 interior tiles, b_rem = 2
    A, B, _ = _pair(5, n=n, b=b)
    Ad, Bd = reference.reconstruct(A), reference.reconstruct(B)
    mb = 3 * b
    Ai, uA, vAt, gA = Ad[:mb, :mb], Ad[:mb, mb:], Ad[mb:, :mb], Ad[mb:, mb:]
    Bi, uB, vBt, gB = Bd[:mb, :mb], Bd[:mb, mb:], Bd[mb:, :mb], Bd[mb:, mb:]
    C = reference.gemm_reference(1.0, "N", A, "N", B, 0.0, None)
    assert np.allclose(C[:mb, :mb], Ai @ Bi + uA @ vBt, atol=1e-13)
    assert np.allclose(C[:mb, mb:], Ai @ uB + uA @ gB, atol=1e-13)
    assert np.allclose(C[mb:, :mb], vAt @ Bi + gA @ vBt, atol=1e-13)
    assert np.allclose(C[mb:, mb:], vAt @ uB + gA @ gB, atol=1e-13)
    # the boundary panels of the TLR matrix are its last tile row / column
    assert tile_sizes(n, b)[-1] == n - mb


def test_linearity():
    A, B, C = _pair(6)
    full = reference.gemm_reference(2.5, "T", A, "N", B, -0.75, C)
    base = reference.gemm_reference(1.0, "T", A, "N", B, 0.0, None)
    assert reference.rel_fro(full - (-0.75) * C, 2.5 * base) <= 1e-14


def _loops_gemm(X, Y):
    m, k = X.shape
    n = Y.shape[1]
    out = np.zeros((m, n))
    for r in range(m):
        for c in range(n):
            s = 0.0
            for t in range(k):
                s += float(X[r, t]) * float(Y[t, c])
            out[r, c] = s
    return out


def test_single_tile_is_dense_gemm():
    rng = np.random.default_rng(7)
    A = random_tlr(rng, 6, 6, 8, has_diag=True, scale=1.0)   # q = 1, only the diagonal
    B = random_tlr(rng, 6, 6, 8, has_diag=True, scale=1.0)
    got = reference.gemm_reference(1.0, "N", A, "N", B, 0.0, None)
    assert np.allclose(got, _loops_gemm(A.diag[0], B.diag[0]), atol=1e-13)


def test_block_diagonal_when_offdiag_ranks_zero():
    rng = np.random.default_rng(8)
    A = random_tlr(rng, 10, 10, 4, rank_lo=0, rank_hi=0, has_diag=True, scale=1.0)
    B = random_tlr(rng, 10, 10, 4, rank_lo=0, rank_hi=0, has_diag=True, scale=1.0)
    C = rng.standard_normal((10, 10))
    got = reference.gemm_reference(2.0, "N", A, "N", B, 0.5, C)
    exp = 0.5 * C
    o = reference.offsets(A.row_sizes)
    for i, s in enumerate(A.row_sizes):
        blk = _loops_gemm(A.diag[i], B.diag[i])
        exp[o[i]:o[i] + s, o[i]:o[i] + s] += 2.0 * blk
    assert np.allclose(got, exp, atol=1e-13)


def _identity_tlr(M: np.ndarray, b: int) -> TLRTiles:
    """Every tile full rank with U = I and V = tile^T: rebuilds M exactly."""
    n = M.shape[0]
    sz = tile_sizes(n, b)
    o = reference.offsets(sz)
    q = len(sz)
    R = np.zeros((q, q), dtype=np.int32)
    U, V = {}, {}
    for i in range(q):
        for j in range(q):
            blk = M[o[i]:o[i] + sz[i], o[j]:o[j] + sz[j]]
            r = sz[i]
            R[i, j] = r
            U[(i, j)] = np.eye(sz[i])
            V[(i, j)] = blk.T.copy()
    return TLRTiles(n, n, b, R, None, U, V, "f64")


def test_full_rank_identity_factors_is_textbook_gemm():
    rng = np.random.default_rng(9)
    Ma, Mb = rng.standard_normal((7, 7)), rng.standard_normal((7, 7))
    A, B = _identity_tlr(Ma, 3), _identity_tlr(Mb, 3)
    got = reference.gemm_reference(1.0, "N", A, "T", B, 0.0, None)
    assert np.allclose(got, _loops_gemm(Ma, Mb.T), atol=1e-12)


@pytest.mark.parametrize("opA,opB", [("N", "N"), ("T", "N"), ("N", "T")])
def test_sampled_block_matches_full(opA, opB):
    A, B, C = _pair(10, n=17, b=5)
    full = reference.gemm_reference(1.5, opA, A, opB, B, 0.25, C)
    rows, cols = (5, 12), (10, 17)
    blk = reference.gemm_reference_block(1.5, opA, A, opB, B, 0.25,
                                         C[rows[0]:rows[1], cols[0]:cols[1]], rows, cols)
    assert np.allclose(blk, full[rows[0]:rows[1], cols[0]:cols[1]], atol=1e-13)
    rng = np.random.default_rng(11)
    Bd = rng.standard_normal((17, 17))
    full = reference.gemm_reference(1.5, opA, A, opB, Bd, 0.25, C)
    blk = reference.gemm_reference_block(1.5, opA, A, opB, Bd, 0.25,
                                         C[rows[0]:rows[1], cols[0]:cols[1]], rows, cols)
    assert np.allclose(blk, full[rows[0]:rows[1], cols[0]:cols[1]], atol=1e-13)

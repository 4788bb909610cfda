"""The TLR-output oracle (oracle/recompress.py) pinned to closed forms.

* Truncation ranks of hand-chosen singular value lists, counted by hand
  (tail energy against tol times the Frobenius norm, equality meeting it).
* A 2 x 2 tile whose singular values follow from its trace and determinant
  (sigma^2 = (T +- sqrt(T^2 - 4 D^2)) / 2): the rank-1 truncation's error is
  the smaller singular value (Eckart-Young).
* A matrix built from prescribed singular values and random orthogonal
  factors: the chosen rank and the truncation error are the closed-form ones.
* Tiles generated with exact ranks are compressed back to those ranks and
  rebuild the matrix to rounding.
* The TLR-output product keeps the diagonal tiles of the exact product, meets
  tol tile by tile, and ignores C (even NaN factors) when beta = 0.
* Planted mistakes in the oracle make these pins fail."""
import math

import numpy as np
import pytest

from oracle import recompress as rc
from oracle import reference
from tlr_inputs import random_tlr

SIG = [8.0, 4.0, 2.0, 1.0, 0.5]        # squares 64, 16, 4, 1, 0.25: Frobenius^2 = 85.25


@pytest.mark.parametrize("tol,rank", [(0.0, 5), (0.05, 5), (0.1, 4), (0.2, 3), (0.5, 1), (1.0, 0)])
def test_truncation_rank_by_hand(tol, rank):
    # limit = (tol * sqrt(85.25))^2 = 85.25 tol^2:  0.05 -> 0.213 (< 0.25), 0.1 -> 0.8525 (0.25 fits, +1 does
    # not), 0.2 -> 3.41 (0.25 + 1 fit, +4 does not), 0.5 -> 21.3125 (0.25+1+4+16 = 21.25 fits), 1.0 -> all
    assert rc.truncation_rank(np.array(SIG), math.sqrt(85.25), tol) == rank


def test_truncation_rank_equality_meets_the_tolerance():
    # sigma = (4, 3), Frobenius 5: tol 0.6 -> limit 9 = 3^2 exactly -> rank 1; tol 0.59 -> rank 2
    assert rc.truncation_rank(np.array([4.0, 3.0]), 5.0, 0.6) == 1
    assert rc.truncation_rank(np.array([4.0, 3.0]), 5.0, 0.59) == 2


def test_two_by_two_tile_closed_form():
    X = np.array([[3.0, 0.0], [4.0, 5.0]])      # T = 50, D = 15: sigma^2 = 45, 5
    U, V, r, s = rc.truncate_tile(X, 0.32)       # sqrt(5/50) = 0.316 <= 0.32
    assert r == 1
    assert np.allclose(s, [math.sqrt(45.0), math.sqrt(5.0)], rtol=1e-14)
    assert abs(np.linalg.norm(X - U @ V.T) - math.sqrt(5.0)) < 1e-13
    U, V, r, _ = rc.truncate_tile(X, 0.31)
    assert r == 2 and np.allclose(U @ V.T, X, atol=1e-14)


def test_prescribed_singular_values():
    rng = np.random.default_rng(3)
    sig = np.array([10.0, 5.0, 1.0, 0.1, 0.01])
    Q1, _ = np.linalg.qr(rng.standard_normal((40, 5)))
    Q2, _ = np.linalg.qr(rng.standard_normal((30, 5)))
    X = (Q1 * sig) @ Q2.T
    # ||sigma|| = sqrt(126.0101); tol 0.01 -> limit 0.1123: 0.01 and 0.1 fit (tail sqrt(0.0101)), 1 does not
    U, V, r, s = rc.truncate_tile(X, 0.01)
    assert r == 3
    assert abs(np.linalg.norm(X - U @ V.T) - math.sqrt(0.0101)) < 1e-12
    assert np.allclose(s[:5], sig, rtol=1e-12)


@pytest.mark.parametrize("n,b,diag", [(60, 16, True), (50, 16, False), (37, 10, True)])
def test_generated_ranks_are_recovered(n, b, diag):
    rng = np.random.default_rng(n + b)
    t = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=6, has_diag=diag, scale=1.0)
    X = reference.reconstruct(t)
    c = rc.compress(X, b, diag, 1e-12)
    assert np.array_equal(c.ranks, t.ranks)
    assert reference.rel_fro(reference.reconstruct(c), X) <= 1e-13


def _product_case(seed=5, n=48, b=16, beta=0.5):
    rng = np.random.default_rng(seed)
    A = random_tlr(rng, n, n, b, rank_lo=1, rank_hi=5, has_diag=True, scale=1.0)
    B = random_tlr(rng, n, n, b, rank_lo=1, rank_hi=5, has_diag=True, scale=1.0)
    C = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=4, has_diag=True, scale=1.0)
    return A, B, C, beta


@pytest.mark.parametrize("tol", [1e-12, 1e-3, 0.3])
def test_tlr_output_meets_tol_and_keeps_the_diagonal(tol):
    A, B, C, beta = _product_case()
    out = rc.tlr_output_reference(0.75, "N", A, "T", B, beta, C, tol)
    X = reference.gemm_reference(0.75, "N", A, "T", B, beta, reference.reconstruct(C))
    err = rc.tile_errors(out, X)
    off = ~np.isnan(err)
    assert np.all(err[off] <= tol * (1 + 1e-12) + 1e-15)
    off0 = reference.offsets(out.row_sizes)
    for i, s in enumerate(out.row_sizes):
        assert np.array_equal(out.diag[i], X[off0[i]:off0[i] + s, off0[i]:off0[i] + s])
    # a looser tolerance never needs a larger rank
    looser = rc.tlr_output_reference(0.75, "N", A, "T", B, beta, C, 2 * tol)
    assert np.all(looser.ranks <= out.ranks)


def test_tlr_output_beta_zero_ignores_c():
    A, B, C, _ = _product_case(seed=6)
    bad = random_tlr(np.random.default_rng(1), C.rows, C.cols, C.b, has_diag=True)
    for key in bad.U:
        bad.U[key] = np.full_like(bad.U[key], np.nan)
    bad.diag = [np.full_like(d, np.nan) for d in bad.diag]
    got = rc.tlr_output_reference(1.0, "N", A, "N", B, 0.0, bad, 1e-6)
    ref = rc.compress(reference.gemm_reference(1.0, "N", A, "N", B, 0.0, None), C.b, True, 1e-6)
    assert np.array_equal(got.ranks, ref.ranks)
    assert np.all(np.isfinite(reference.reconstruct(got)))


# ---- planted mistakes --------------------------------------------------------

def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_tail_of_singular_values_not_squared_is_caught(monkeypatch):
    def bad(sigma, fro, tol):
        s = np.asarray(sigma)
        r = len(s)
        tail = 0.0
        for k in range(len(s) - 1, -1, -1):
            if tail + s[k] <= tol * fro:
                tail += s[k]
                r = k
            else:
                break
        return r
    monkeypatch.setattr(rc, "truncation_rank", bad)
    _fails(test_truncation_rank_by_hand, 0.5, 1)     # unsquared: 0.5+1+2 = 3.5 <= 4.62 < 7.5 gives rank 2


def test_strict_inequality_is_caught(monkeypatch):
    def bad(sigma, fro, tol):
        s = np.asarray(sigma)
        limit = (tol * fro) ** 2
        r, tail = len(s), 0.0
        for k in range(len(s) - 1, -1, -1):
            if tail + s[k] * s[k] < limit:
                tail += s[k] * s[k]
                r = k
            else:
                break
        return r
    monkeypatch.setattr(rc, "truncation_rank", bad)
    _fails(test_truncation_rank_equality_meets_the_tolerance)


def test_truncated_diagonal_is_caught(monkeypatch):
    orig = rc.compress

    def bad(X, b, has_diag, tol):
        return orig(X, b, False, tol) if has_diag else orig(X, b, has_diag, tol)
    monkeypatch.setattr(rc, "compress", bad)
    with pytest.raises((AssertionError, TypeError, AttributeError)):
        test_tlr_output_meets_tol_and_keeps_the_diagonal(1e-3)


def test_unscaled_singular_vectors_are_caught(monkeypatch):
    def bad(X, tol):
        X = np.asarray(X, dtype=np.float64)
        Us, s, Vt = np.linalg.svd(X, full_matrices=False)
        r = rc.truncation_rank(s, float(np.linalg.norm(X)), tol)
        return Us[:, :r], Vt[:r, :].T.copy(), r, s
    monkeypatch.setattr(rc, "truncate_tile", bad)
    _fails(test_two_by_two_tile_closed_form)

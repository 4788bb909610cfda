"""The dense oracle agrees with the per-k tile loop on tiny grids.

The tile loop (oracle.brute) evaluates every (i, k, j) term with explicit
scalar loops and never forms a dense operand; the reference (oracle.reference)
rebuilds every tile and multiplies once with BLAS.  Agreement to 1e-13
relative pins tile placement, boundary tiles, op handling, the diagonal
terms and the alpha/beta update of the reference."""
import itertools

import numpy as np
import pytest

from oracle import brute, reference
from tlr_inputs import random_tlr


def _case(seed, n, b, opA, opB, beta, dense_b=False, diag=True, rank_lo=0):
    rng = np.random.default_rng(seed)
    A = random_tlr(rng, n, n, b, rank_lo=rank_lo, has_diag=diag, scale=1.0)
    if dense_b:
        B = rng.standard_normal((n, n))
    else:
        B = random_tlr(rng, n, n, b, rank_lo=rank_lo, has_diag=diag, scale=1.0)
    C = np.full((n, n), np.nan) if beta == 0.0 else rng.standard_normal((n, n))
    alpha = 0.75
    ref = reference.gemm_reference(alpha, opA, A, opB, B, beta, C)
    for assoc in ("right", "left"):
        bf, _ = brute.tile_loop(alpha, opA, A, opB, B, beta, C, assoc)
        assert np.all(np.isfinite(ref))
        assert reference.rel_fro(bf, ref) <= 1e-13, (seed, n, b, opA, opB, beta, assoc)


GRID = [(q, b, rem) for q in (1, 2, 3, 4) for b in (2, 3, 5, 8) for rem in (0, 1, 3) if rem < b]


@pytest.mark.parametrize("q,b,rem", GRID)
def test_tlr_tlr_all_ops(q, b, rem):
    n = q * b if rem == 0 else (q - 1) * b + rem
    for t, (opA, opB, beta) in enumerate(itertools.product("NT", "NT", (0.0, 0.5, 1.0))):
        _case(100 * q + 10 * b + rem + 1000 * t, n, b, opA, opB, beta)


@pytest.mark.parametrize("q,b,rem", [(3, 4, 0), (3, 5, 2), (4, 3, 1), (1, 6, 0)])
def test_tlr_dense(q, b, rem):
    n = q * b if rem == 0 else (q - 1) * b + rem
    for t, (opA, opB, beta) in enumerate(itertools.product("NT", "NT", (0.0, 0.5))):
        _case(7 + t, n, b, opA, opB, beta, dense_b=True)


def test_no_diagonal_and_rectangular_grid():
    # worked-example shape class: a 2x3 grid times a 3x3 grid, no dense diagonal
    rng = np.random.default_rng(5)
    A = random_tlr(rng, 8, 12, 4, rank_lo=0, has_diag=False, scale=1.0)
    B = random_tlr(rng, 12, 12, 4, rank_lo=0, has_diag=False, scale=1.0)
    ref = reference.gemm_reference(1.0, "N", A, "N", B, 0.0, None)
    for assoc in ("right", "left"):
        bf, _ = brute.tile_loop(1.0, "N", A, "N", B, 0.0, None, assoc)
        assert reference.rel_fro(bf, ref) <= 1e-13

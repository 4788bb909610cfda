"""The per-contraction-tile loop (TLR_PLAN_PER_K, the comparator of "Many
small GEMMs": one coupling, right product and update per output tile and
contraction tile, one pass over C per k) on the GPU against the oracle: every
op pair, beta in {0 (NaN-filled C), 0.7}, with and without dense diagonals,
ragged tails, fp64 and fp32; and operands padded with zero columns to one
common rank (the batched-GEMM form) give the same product.
Bar: relative Frobenius error <= 1e-12 (fp64), <= 1e-5 (fp32)."""
import itertools

import numpy as np
import pytest

from gpu_helpers import TOL, check_tlr, gpu_ready, padded_tlr, run_tlr, say
from oracle import reference
from tlr_inputs import random_tlr

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ready(), reason="needs the GPU and libtlrgemm.so")]

PER_K = 0x20


@pytest.mark.parametrize("n,b", [(256, 64), (200, 64), (130, 32)])
@pytest.mark.parametrize("opA,opB", [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")])
def test_per_k_ops(n, b, opA, opB):
    for t, (beta, diag) in enumerate(itertools.product((0.0, 0.7), (True, False))):
        rng = np.random.default_rng(5 * n + b + 100 * t)
        A = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=20, has_diag=diag)
        B = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=20, has_diag=diag)
        C = rng.standard_normal((n, n))
        say(f"per-k n={n} b={b} {opA}{opB} beta={beta} diag={diag}")
        check_tlr(A, B, opA, opB, 1.25, beta, None if beta == 0 else C, flags=PER_K)


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_per_k_padded_equals_ragged(dtype):
    rng = np.random.default_rng(44)
    A = random_tlr(rng, 300, 300, 64, rank_lo=1, rank_hi=24, has_diag=True, dtype=dtype)
    B = random_tlr(rng, 300, 300, 64, rank_lo=1, rank_hi=24, has_diag=True, dtype=dtype)
    C = rng.standard_normal((300, 300))
    rmax = int(max(A.ranks.max(), B.ranks.max()))
    Ap, Bp = padded_tlr(A, rmax), padded_tlr(B, rmax)
    say(f"per-k padded {dtype} rmax={rmax}")
    ref = reference.gemm_reference(1.0, "N", A, "N", B, 1.0, C)
    for (x, y) in ((A, B), (Ap, Bp)):
        got = run_tlr(x, y, "N", "N", 1.0, 1.0, C, flags=PER_K)
        assert reference.rel_fro(got, ref) <= TOL[dtype]

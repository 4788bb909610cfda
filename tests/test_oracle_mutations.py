"""Planted mistakes in the oracle are caught by its pins.

Each test patches one plausible bug into an oracle function (on the CPU, for
the duration of the test only) and checks that the corresponding pin fails:
a dropped diagonal term, an ignored transpose, a transposed tile placement,
C read when beta = 0, alpha applied to C, column sums used for rho, and a
dropped coupling term in the flop count."""
import json
import os

import numpy as np

from oracle import brute, plan_arith as pa, reference
from tlr_inputs import random_tlr, tile_sizes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _brute_agrees(opA="N", opB="N", beta=0.5, n=10, b=4, seed=3):
    rng = np.random.default_rng(seed)
    A = random_tlr(rng, n, n, b, rank_lo=1, has_diag=True, scale=1.0)
    B = random_tlr(rng, n, n, b, rank_lo=1, has_diag=True, scale=1.0)
    C = rng.standard_normal((n, n))
    ref = reference.gemm_reference(0.75, opA, A, opB, B, beta, C)
    bf, _ = brute.tile_loop(0.75, opA, A, opB, B, beta, C, "right")
    return reference.rel_fro(bf, ref) <= 1e-13


def test_unpatched_agrees():
    assert _brute_agrees() and _brute_agrees("T", "T")


def test_dropped_diagonal_is_caught(monkeypatch):
    orig = reference.dense_tile

    def bad(t, i, j):
        out = orig(t, i, j)
        return np.zeros_like(out) if (t.has_diag and i == j) else out
    monkeypatch.setattr(reference, "dense_tile", bad)
    assert not _brute_agrees()


def test_ignored_transpose_is_caught(monkeypatch):
    monkeypatch.setattr(reference, "_op", lambda M, op: M)
    assert not _brute_agrees("T", "N")


def test_transposed_tile_placement_is_caught(monkeypatch):
    orig = reference.dense_tile

    def bad(t, i, j):
        if t.has_diag and i == j:
            return orig(t, i, j)
        out = orig(t, j, i) if (t.row_sizes[i] == t.row_sizes[j]) else orig(t, i, j)
        return out
    monkeypatch.setattr(reference, "dense_tile", bad)
    assert not _brute_agrees(n=12, b=4)


def test_beta_zero_reading_c_is_caught(monkeypatch):
    def bad(alpha, opA, A, opB, B, beta, C_in):
        Ad = reference._op(reference.reconstruct(A), opA)
        Bd = reference._op(reference.reconstruct(B), opB)
        return alpha * (Ad @ Bd) + beta * np.asarray(C_in)
    monkeypatch.setattr(reference, "gemm_reference", bad)
    rng = np.random.default_rng(1)
    A = random_tlr(rng, 8, 8, 4, has_diag=True)
    B = random_tlr(rng, 8, 8, 4, has_diag=True)
    got = reference.gemm_reference(1.0, "N", A, "N", B, 0.0, np.full((8, 8), np.nan))
    assert not np.all(np.isfinite(got))


def test_alpha_on_c_is_caught(monkeypatch):
    orig = reference.gemm_reference

    def bad(alpha, opA, A, opB, B, beta, C_in):
        return alpha * orig(1.0, opA, A, opB, B, beta, C_in)
    monkeypatch.setattr(reference, "gemm_reference", bad)
    assert not _brute_agrees()


def test_rho_from_column_sums_is_caught(monkeypatch):
    monkeypatch.setattr(pa, "rho", lambda RA: [int(x) for x in np.asarray(RA).sum(axis=0)])
    RA = np.array(GOLD["A_ranks"])
    assert pa.rho(RA) != GOLD["printed"]["rho"]


def test_dropped_coupling_flops_is_caught():
    rng = np.random.default_rng(2)
    A = random_tlr(rng, 9, 9, 3, rank_lo=1, has_diag=True, scale=1.0)
    B = random_tlr(rng, 9, 9, 3, rank_lo=1, has_diag=True, scale=1.0)
    s = tile_sizes(9, 3)
    _, flops = brute.tile_loop(1.0, "N", A, "N", B, 0.0, None, "right")
    good = pa.useful_flops(A.ranks, B.ranks, s, s, s, True, True, "right")
    coupling = sum(2 * a * c * d for (_, _, _, (a, c, d)) in pa.coupling_products(A.ranks, B.ranks, s))
    assert flops == good and flops != good - coupling

"""Planted mistakes in the oracle make its pins fail.

Each test patches one plausible bug into an oracle function (on the CPU, for
the duration of the test only), then runs the pin that is meant to catch it
(a test function of tests/test_oracle_*.py, called directly) and requires
that pin to fail with an AssertionError.  The unpatched pins pass in their
own modules.  Planted mistakes: a dropped diagonal tile, an ignored
transpose, a transposed tile placement, C read when beta = 0, alpha applied
to C, column sums taken for rho, a dropped coupling term in the flop count,
and a diagonal-term workspace sized by the wrong tile list."""
import numpy as np
import pytest

import test_oracle_brute as pin_brute
import test_oracle_invariants as pin_inv
import test_oracle_plan_arith as pin_arith
from oracle import plan_arith as pa
from oracle import reference


def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_dropped_diagonal_is_caught(monkeypatch):
    orig = reference.dense_tile

    def bad(t, i, j):
        out = orig(t, i, j)
        return np.zeros_like(out) if (t.has_diag and i == j) else out
    monkeypatch.setattr(reference, "dense_tile", bad)
    _fails(pin_brute.test_tlr_tlr_all_ops, 3, 4, 0)
    _fails(pin_inv.test_block_diagonal_when_offdiag_ranks_zero)


def test_ignored_transpose_is_caught(monkeypatch):
    monkeypatch.setattr(reference, "_op", lambda M, op: M)
    _fails(pin_brute.test_tlr_tlr_all_ops, 2, 3, 0)
    _fails(pin_inv.test_transpose_by_factor_swap, "T", "N")


def test_transposed_tile_placement_is_caught(monkeypatch):
    orig = reference.dense_tile

    def bad(t, i, j):
        if (t.has_diag and i == j) or t.row_sizes[i] != t.row_sizes[j]:
            return orig(t, i, j)
        return orig(t, j, i)
    monkeypatch.setattr(reference, "dense_tile", bad)
    _fails(pin_brute.test_tlr_tlr_all_ops, 3, 4, 0)


def test_beta_zero_reading_c_is_caught(monkeypatch):
    orig = reference.gemm_reference

    def bad(alpha, opA, A, opB, B, beta, C_in):
        out = orig(alpha, opA, A, opB, B, 1.0 if beta == 0.0 else beta, C_in)
        return out - (np.asarray(C_in) if beta == 0.0 and C_in is not None else 0.0)
    monkeypatch.setattr(reference, "gemm_reference", bad)
    _fails(pin_inv.test_beta_zero_ignores_c, np.nan)


def test_alpha_on_c_is_caught(monkeypatch):
    orig = reference.gemm_reference

    def bad(alpha, opA, A, opB, B, beta, C_in):
        return alpha * orig(1.0, opA, A, opB, B, beta, C_in)
    monkeypatch.setattr(reference, "gemm_reference", bad)
    _fails(pin_brute.test_tlr_tlr_all_ops, 2, 3, 1)
    _fails(pin_inv.test_linearity)


def test_rho_from_column_sums_is_caught(monkeypatch):
    monkeypatch.setattr(pa, "rho", lambda RA: [int(x) for x in np.asarray(RA).sum(axis=0)])
    _fails(pin_arith.test_worked_example, "B_a")
    _fails(pin_arith.test_worked_example, "B_b")


def test_dropped_coupling_flops_is_caught(monkeypatch):
    orig = pa.useful_flops

    def bad(RA, RB, ms, ks, ns, dA, dB, order, I=None, J=None):
        RA_, RB_ = np.asarray(RA), np.asarray(RB)
        I_ = range(RA_.shape[0]) if I is None else I
        J_ = range(RB_.shape[1]) if J is None else J
        coupling = sum(2 * ra * rb * sk for (i, k, j, (ra, rb, sk)) in pa.coupling_products(RA_, RB_, ks)
                       if i in I_ and j in J_ and not (dA and i == k) and not (dB and k == j))
        return orig(RA, RB, ms, ks, ns, dA, dB, order, I, J) - coupling
    monkeypatch.setattr(pa, "useful_flops", bad)
    _fails(pin_arith.test_brute_force_flops_equal_useful_flops, 1, 9, 3, True, "N", "N")
    _fails(pin_arith.test_uniform_rank_closed_form, 3, 8, 2, 5)


def test_diagonal_workspace_with_wrong_sizes_is_caught(monkeypatch):
    orig = pa.workspace_elements

    def bad(RA, RB, ms, ks, ns, dA, dB, order, I, J):
        # X_i = D_A,ii W_{i,J} sized with the column tile list instead of the row one
        w = orig(RA, RB, ms, ks, ns, dA, dB, order, I, J)
        if order == "right" and dA:
            w["diag"] = sum(ns[i] * sum(int(np.asarray(RB)[i, j]) for j in J) for i in I)
        return w
    monkeypatch.setattr(pa, "workspace_elements", bad)
    _fails(pin_arith.test_workspace_elements_hand_counts, pin_arith.WS_R, "right")

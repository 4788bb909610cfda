"""Exhaustive self-check of the launch descriptors on the CPU (TLR_PLAN_VALIDATE).

For every plan below the library replays its launches on per-element state
and refuses the plan unless: every operand and output range lies inside its
buffer; writes inside one launch never overlap; every workspace element a
launch reads was written by an earlier launch of the same rectangle; every
element of C is written exactly once and C's padding rows never.  Together
with the bounds check that runs on every plan, this is what shows, before any
kernel runs, that the grouped GEMM stays inside its buffers."""
import itertools

import numpy as np
import pytest

from hpc_linear_algebra_amd import tlrgemm as T
from tlr_inputs import CONFIGS, config_ranks, tile_sizes

V = T.TLR_PLAN_VALIDATE


def _ranks(rng, q, sz, diag, lo, hi):
    R = rng.integers(lo, hi + 1, size=(q, q)).astype(np.int32)
    R = np.minimum(R, np.minimum.outer(sz, sz)).astype(np.int32)
    if diag:
        np.fill_diagonal(R, 0)
    return R


CASES = [(n, b) for n in (64, 200, 300, 513) for b in (16, 64, 128)]


@pytest.mark.parametrize("n,b", CASES)
def test_random_plans_validate(n, b):
    rng = np.random.default_rng(n * 1000 + b)
    sz = tile_sizes(n, b)
    q = len(sz)
    for diag, (opA, opB), flags, ns in itertools.product(
            (True, False), [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")],
            (0, T.TLR_PLAN_FORCE_RIGHT, T.TLR_PLAN_FORCE_LEFT), (1, 3)):
        RA = _ranks(rng, q, sz, diag, 0, 20)
        RB = _ranks(rng, q, sz, diag, 0, 20)
        A, B = T.Shape(n, n, b, RA, diag), T.Shape(n, n, b, RB, diag)
        full = T.tlr_plan_info(T.tlr_gemm_analyze("f64", opA, A, opB, B, ldc=n + 3, n_streams=ns,
                                                  flags=flags))["workspace_bytes"]
        for frac in (0, 0.3):
            budget = int(full * frac)
            try:
                T.tlr_gemm_analyze("f64", opA, A, opB, B, ldc=n + 3, workspace_budget=budget,
                                   n_streams=ns, flags=flags | V)
            except T.TLRError as e:
                assert e.status == T.TLR_ERR_WORKSPACE, str(e)
        if diag:
            for ncols in (1, n + 9):
                dr, dc = (n, ncols) if opB == "N" else (ncols, n)
                T.tlr_gemm_analyze("f32", opA, A, opB, None, dr, dc, ldb=dr + 2, ldc=n, flags=V)


@pytest.mark.parametrize("c", [1, 2, 3])
def test_workload_plans_validate(c):
    cfg = CONFIGS[c]
    N, b = cfg["N"], cfg["b"]
    A = T.Shape(N, N, b, config_ranks(c, 0), True)
    if cfg["kind"] == "tlr_dense":
        T.tlr_gemm_analyze(cfg["dtype"], cfg["opA"], A, cfg["opB"], None, N, N, N, N, flags=V)
    else:
        B = T.Shape(N, N, b, config_ranks(c, 1), True)
        T.tlr_gemm_analyze(cfg["dtype"], cfg["opA"], A, cfg["opB"], B, ldc=N, flags=V)


def test_boundary_workload_structure_validates():
    # the workload-4 structure scaled down: 12 x 12 tiles with a 184 remainder,
    # uniform ranks in [16, 128], a budget that forces several rectangles
    rng = np.random.default_rng(4)
    N, b = 11 * 256 + 184, 256
    sz = tile_sizes(N, b)
    RA, RB = _ranks(rng, len(sz), sz, True, 16, 128), _ranks(rng, len(sz), sz, True, 16, 128)
    A, B = T.Shape(N, N, b, RA, True), T.Shape(N, N, b, RB, True)
    for ns in (1, 4):
        w = T.tlr_gemm_workspace_bytes("f32", "N", A, "N", B, n_streams=ns, runs=8)
        p = T.tlr_gemm_analyze("f32", "N", A, "N", B, ldc=N, workspace_budget=w, n_streams=ns, flags=V)
        assert T.tlr_plan_info(p)["runs"] >= 2


def test_pipelined_plans_validate():
    rng = np.random.default_rng(9)
    for n, b in ((640, 64), (1000, 128), (513, 32)):
        sz = tile_sizes(n, b)
        RA, RB = _ranks(rng, len(sz), sz, True, 1, 24), _ranks(rng, len(sz), sz, True, 1, 24)
        A, B = T.Shape(n, n, b, RA, True), T.Shape(n, n, b, RB, True)
        for budget in (0, 2_000_000):
            p = T.tlr_gemm_analyze("f64", "T", A, "N", B, ldc=n, workspace_budget=budget, n_streams=2,
                                   flags=T.TLR_PLAN_PIPELINE | V)
            info = T.tlr_plan_info(p)
            assert info["groups"] == 2 and info["runs"] >= 2
            if budget:
                assert info["workspace_bytes"] <= budget
    with pytest.raises(T.TLRError):
        T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n, n_streams=1, flags=T.TLR_PLAN_PIPELINE)

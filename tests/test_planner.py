"""Host planner behind the C ABI, pinned to the oracle's rank arithmetic.

* Worked example of "Tile-Low-Rank GEMM: Designing Storage Around the
  Contraction" (fixture tests/golden/worked_example.json): the planner's
  Stage-1 and Stage-3 GEMM shapes, final-stage costs and order choice.
* Useful flops of both association orders equal the oracle's term-by-term
  count exactly (integers), for random grids, op combinations, dense B and
  the five workloads' rank tables.
* Schedules under a budget: every output tile in exactly one rectangle, every
  rectangle within the budget and at least the oracle's element count of its
  intermediates, the cheaper feasible order, and the runs -> budget inversion.
"""
import json
import os

import numpy as np
import pytest

from hpc_linear_algebra_amd import tlrgemm as T
from oracle import checks, plan_arith as pa
from tlr_inputs import CONFIGS, config_ranks, tile_sizes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


@pytest.mark.parametrize("cand", sorted(GOLD["B_ranks_candidates"]))
def test_worked_example(cand):
    b = GOLD["b"]
    RA = np.array(GOLD["A_ranks"], dtype=np.int32)
    RB = np.array(GOLD["B_ranks_candidates"][cand], dtype=np.int32)
    A = T.Shape(2 * b, 3 * b, b, RA, False)
    B = T.Shape(3 * b, 3 * b, b, RB, False)
    p = T.tlr_gemm_analyze("f32", "N", A, "N", B, ldc=2 * b)
    info = T.tlr_plan_info(p)
    P = GOLD["printed"]
    assert info["runs"] == 1
    r = T.tlr_plan_rect(p, 0)
    assert (r["i0"], r["i1"], r["j0"], r["j1"]) == (0, 2, 0, 3)
    assert r["order"] == T.TLR_ORDER_RIGHT
    assert [list(x) for x in T.tlr_plan_stage_shapes(p, 0, 1)] == P["stage1_shapes_MNK"]
    assert [list(x) for x in T.tlr_plan_stage_shapes(p, 0, 3)] == P["stage3_right_shapes_MNK"]
    assert info["final_flops_right"] == 2 * b * b * P["F_R_over_2b2"]
    assert info["final_flops_left"] == 2 * b * b * P["F_L_over_2b2"]
    s = [b] * 3
    assert info["flops_right"] == pa.useful_flops(RA, RB, [b, b], s, s, False, False, "right")
    assert info["flops_left"] == pa.useful_flops(RA, RB, [b, b], s, s, False, False, "left")
    # three grouped launches per rectangle (the right product's three tasks
    # with rank(B_kj) <= 16 are too few for a strip launch of their own)
    assert info["launches"] == 3
    stages = [T.tlr_plan_launch(p, l)["stage"] for l in range(3)]
    assert stages == [1, 2, 3]


def _rand_ranks(rng, q, b, diag, lo=0, hi=None):
    hi = b if hi is None else hi
    R = rng.integers(lo, hi + 1, size=(q, q)).astype(np.int32)
    if diag:
        np.fill_diagonal(R, 0)
    return R


def test_strip_split():
    """Right/left-product tasks with K <= 16 (here rank(A_ik) <= 16, left order)
    go to a strip launch of 128 x 512 blocks after the grouped launch of the
    others, when they make at least 512 blocks; 16-bit plans and small grids
    keep one launch."""
    rng = np.random.default_rng(11)
    q, b = 24, 256
    RA = _rand_ranks(rng, q, b, True, lo=0, hi=24)
    RB = _rand_ranks(rng, q, b, True, lo=1, hi=24)
    A, B = T.Shape(q * b, q * b, b, RA, True), T.Shape(q * b, q * b, b, RB, True)
    flags = T.TLR_PLAN_FORCE_LEFT | T.TLR_PLAN_VALIDATE
    p = T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=q * b, flags=flags)
    L = [T.tlr_plan_launch(p, l) for l in range(T.tlr_plan_info(p)["launches"])]
    st2 = [x for x in L if x["stage"] == 2]
    SN = RB.sum(axis=1)          # coupling columns of contraction tile k
    tasks = [(i, k) for i in range(q) for k in range(q) if k != i and SN[k] > 0]
    small = [(i, k) for (i, k) in tasks if RA[i, k] <= 16]
    assert [x["tasks"] for x in st2] == [len(tasks) - len(small), len(small)]
    blocks = sum(2 * -(-int(SN[k]) // 512) for (_, k) in small)
    assert blocks >= 512
    assert st2[1]["workgroups"] >= blocks and st2[1]["workgroups"] % 8 == 0
    assert st2[1]["useful_flops"] == sum(2.0 * b * SN[k] * RA[i, k] for (i, k) in small)
    A8, B8 = (T.Shape(q * b, q * b, b, (R + 7) // 8 * 8, True) for R in (RA, RB))   # 16-bit: ranks of 8
    p16 = T.tlr_gemm_analyze("f16", "N", A8, "N", B8, ldc=q * b, flags=flags)
    assert sum(T.tlr_plan_launch(p16, l)["stage"] == 2 for l in range(T.tlr_plan_info(p16)["launches"])) == 1
    A4, B4 = (T.Shape(4 * b, 4 * b, b, R[:4, :4].copy(), True) for R in (RA, RB))
    p4 = T.tlr_gemm_analyze("f64", "N", A4, "N", B4, ldc=4 * b, flags=flags)
    assert sum(T.tlr_plan_launch(p4, l)["stage"] == 2 for l in range(T.tlr_plan_info(p4)["launches"])) == 1


CASES = [(0, 5, 4, 0, True), (1, 4, 3, 2, True), (2, 3, 5, 4, False), (3, 6, 2, 1, True), (4, 1, 8, 0, True),
         (5, 7, 6, 3, False)]


@pytest.mark.parametrize("seed,q,b,rem,diag", CASES)
@pytest.mark.parametrize("opA,opB", [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")])
def test_useful_flops_match_oracle(seed, q, b, rem, diag, opA, opB):
    rng = np.random.default_rng(seed)
    n = q * b if rem == 0 else (q - 1) * b + rem
    sz = tile_sizes(n, b)
    RA = _rand_ranks(rng, q, b, diag)
    RB = _rand_ranks(rng, q, b, diag)
    RA = np.minimum(RA, np.minimum.outer(sz, sz)).astype(np.int32)
    RB = np.minimum(RB, np.minimum.outer(sz, sz)).astype(np.int32)
    p = T.tlr_gemm_analyze("f64", opA, T.Shape(n, n, b, RA, diag), opB, T.Shape(n, n, b, RB, diag), ldc=n)
    info = T.tlr_plan_info(p)
    oA, oB = pa.op_ranks(RA, opA), pa.op_ranks(RB, opB)
    fr = pa.useful_flops(oA, oB, sz, sz, sz, diag, diag, "right")
    fl = pa.useful_flops(oA, oB, sz, sz, sz, diag, diag, "left")
    assert info["flops_right"] == fr
    assert info["flops_left"] == fl
    assert info["useful_flops"] == min(fr, fl)
    assert info["final_flops_right"] == pa.final_stage_flops(oA, oB, sz, sz, "right")
    assert info["final_flops_left"] == pa.final_stage_flops(oA, oB, sz, sz, "left")
    launches = [T.tlr_plan_launch(p, l) for l in range(info["launches"])]
    assert sum(L["useful_flops"] for L in launches) == info["useful_flops"]
    assert info["executed_flops"] >= info["useful_flops"]
    # dense B
    ncols = n + 3
    dr, dc = (n, ncols) if opB == "N" else (ncols, n)
    pd = T.tlr_gemm_analyze("f64", opA, T.Shape(n, n, b, RA, diag), opB, None, dr, dc, ldb=dr, ldc=n)
    infd = T.tlr_plan_info(pd)
    assert infd["useful_flops"] == pa.useful_flops_dense_b(oA, sz, sz, ncols, diag)


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_workload_flops_and_orders(c):
    cfg = CONFIGS[c]
    N, b = cfg["N"], cfg["b"]
    sz = tile_sizes(N, b)
    RA = config_ranks(c, 0)
    A = T.Shape(N, N, b, RA, True)
    oA = pa.op_ranks(RA, cfg["opA"])
    if cfg["kind"] == "tlr_dense":
        p = T.tlr_gemm_analyze(cfg["dtype"], cfg["opA"], A, cfg["opB"], None, N, N, N, N)
        assert T.tlr_plan_info(p)["useful_flops"] == pa.useful_flops_dense_b(oA, sz, sz, N, True)
        return
    RB = config_ranks(c, 1)
    B = T.Shape(N, N, b, RB, True)
    oB = pa.op_ranks(RB, cfg["opB"])
    p = T.tlr_gemm_analyze(cfg["dtype"], cfg["opA"], A, cfg["opB"], B, ldc=N)
    info = T.tlr_plan_info(p)
    fr = pa.useful_flops(oA, oB, sz, sz, sz, True, True, "right")
    fl = pa.useful_flops(oA, oB, sz, sz, sz, True, True, "left")
    assert (info["flops_right"], info["flops_left"]) == (fr, fl)
    expect = {1: (5.506e7, 5.197e7, "left"), 3: (2.2205e11, 2.2076e11, "left"),
              4: (4.6220e12, 4.6294e12, "right"), 5: (3.4979e12, 3.4701e12, "left")}[c]
    assert abs(fr / expect[0] - 1) < 1e-3 and abs(fl / expect[1] - 1) < 1e-3
    r = T.tlr_plan_rect(p, 0)
    assert r["order"] == (T.TLR_ORDER_LEFT if expect[2] == "left" else T.TLR_ORDER_RIGHT)


def _schedule_invariants(p, qm, qn, budget, RA, RB, sz, diag, es):
    info = T.tlr_plan_info(p)
    rects = [T.tlr_plan_rect(p, r) for r in range(info["runs"])]
    assert checks.covers_exactly_once([(r["i0"], r["i1"], r["j0"], r["j1"]) for r in rects], qm, qn)
    for r in rects:
        I, J = range(r["i0"], r["i1"]), range(r["j0"], r["j1"])
        order = "right" if r["order"] == T.TLR_ORDER_RIGHT else "left"
        w = pa.workspace_elements(RA, RB, sz, sz, sz, diag, diag, order, I, J)
        assert r["ws_bytes"] >= es * sum(w.values())
        if budget:
            assert r["ws_bytes"] <= budget
        # the chosen order is the cheaper one among the orders that fit
        other = "left" if order == "right" else "right"
        wo = pa.workspace_elements(RA, RB, sz, sz, sz, diag, diag, other, I, J)
        if budget == 0 or es * sum(wo.values()) + 256 * 3 * (len(sz) + 2 * len(I) + 2 * len(J)) <= budget:
            assert r["useful_flops"] <= pa.useful_flops(RA, RB, sz, sz, sz, diag, diag, other, I, J) + 0.0
    assert sum(r["useful_flops"] for r in rects) == info["useful_flops"]
    if budget:
        assert info["workspace_bytes"] <= budget
    return rects


@pytest.mark.parametrize("seed,q,b,frac", [(1, 6, 16, 0.5), (2, 8, 8, 0.2), (3, 5, 12, 0.05), (4, 9, 7, 0.3)])
def test_schedule_under_budget(seed, q, b, frac):
    rng = np.random.default_rng(seed)
    n = q * b
    sz = tile_sizes(n, b)
    RA = _rand_ranks(rng, q, b, True, 1, b // 2)
    RB = _rand_ranks(rng, q, b, True, 1, b // 2)
    A, B = T.Shape(n, n, b, RA, True), T.Shape(n, n, b, RB, True)
    full = T.tlr_plan_info(T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n))["workspace_bytes"]
    budget = max(int(full * frac), 1)
    try:
        p = T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n, workspace_budget=budget)
    except T.TLRError as e:
        assert e.status == T.TLR_ERR_WORKSPACE
        return
    rects = _schedule_invariants(p, q, q, budget, RA, RB, sz, True, 8)
    assert len(rects) > 1


@pytest.mark.parametrize("runs", [1, 2, 3, 5, 8])
def test_runs_to_budget(runs):
    rng = np.random.default_rng(11)
    q, b = 6, 16
    n = q * b
    RA = _rand_ranks(rng, q, b, True, 1, 8)
    RB = _rand_ranks(rng, q, b, True, 1, 8)
    A, B = T.Shape(n, n, b, RA, True), T.Shape(n, n, b, RB, True)
    w = T.tlr_gemm_workspace_bytes("f64", "N", A, "N", B, runs=runs)
    p = T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n, workspace_budget=w)
    assert T.tlr_plan_info(p)["runs"] <= runs
    try:
        p2 = T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n, workspace_budget=w - 1)
        assert T.tlr_plan_info(p2)["runs"] > runs
    except T.TLRError as e:
        assert e.status == T.TLR_ERR_WORKSPACE
    if runs == 1:
        full = T.tlr_plan_info(T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n))["workspace_bytes"]
        assert w == full


def test_boundary_regions_on_streams():
    # workload-4 structure (30 x 30 tiles, last tile 304) under its 1 GiB budget
    c = 4
    N, b = CONFIGS[c]["N"], CONFIGS[c]["b"]
    sz = tile_sizes(N, b)
    RA, RB = config_ranks(c, 0), config_ranks(c, 1)
    A, B = T.Shape(N, N, b, RA, True), T.Shape(N, N, b, RB, True)
    budget = 1 << 30
    p = T.tlr_gemm_analyze("f32", "N", A, "N", B, ldc=N, workspace_budget=budget, n_streams=4)
    info = T.tlr_plan_info(p)
    assert info["groups"] == 4
    rects = _schedule_invariants(p, 30, 30, budget, RA, RB, sz, True, 4)
    assert info["runs"] > 4
    # regions are disjoint: interior rectangles stay inside the 29 x 29 block
    for r in rects:
        if r["group"] == 0:
            assert r["i1"] <= 29 and r["j1"] <= 29
        else:
            assert r["i0"] >= 29 or r["j0"] >= 29
    seq = T.tlr_gemm_analyze("f32", "N", A, "N", B, ldc=N, workspace_budget=budget, n_streams=1)
    assert T.tlr_plan_info(seq)["groups"] == 1
    assert T.tlr_plan_info(seq)["useful_flops"] >= info["useful_flops"] * 0.99


def test_forced_orders():
    rng = np.random.default_rng(3)
    q, b = 4, 8
    n = q * b
    RA, RB = _rand_ranks(rng, q, b, True, 1, 4), _rand_ranks(rng, q, b, True, 1, 4)
    A, B = T.Shape(n, n, b, RA, True), T.Shape(n, n, b, RB, True)
    for fl, o in ((T.TLR_PLAN_FORCE_RIGHT, T.TLR_ORDER_RIGHT), (T.TLR_PLAN_FORCE_LEFT, T.TLR_ORDER_LEFT)):
        p = T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n, flags=fl)
        assert all(T.tlr_plan_rect(p, r)["order"] == o for r in range(T.tlr_plan_info(p)["runs"]))


def test_empty_and_degenerate():
    z = np.zeros((0, 0), dtype=np.int32)
    p = T.tlr_gemm_analyze("f64", "N", T.Shape(0, 0, 4, z, True), "N", T.Shape(0, 0, 4, z, True), ldc=1)
    info = T.tlr_plan_info(p)
    assert info["runs"] == 0 and info["launches"] == 0 and info["useful_flops"] == 0
    # every off-diagonal rank zero: block-diagonal product, only D_A D_B work
    R = np.zeros((3, 3), dtype=np.int32)
    p = T.tlr_gemm_analyze("f64", "N", T.Shape(12, 12, 4, R, True), "N", T.Shape(12, 12, 4, R, True), ldc=12)
    assert T.tlr_plan_info(p)["useful_flops"] == 3 * 2 * 4 ** 3


@pytest.mark.parametrize("order", [T.TLR_PLAN_FORCE_RIGHT, T.TLR_PLAN_FORCE_LEFT])
def test_side_launch_holds_the_diagonal_terms(order):
    # with dense diagonal tiles the input-only diagonal products form a side
    # launch (stage 4) between the coupling and the right/left product of each
    # rectangle; its useful flops are exactly those products'
    rng = np.random.default_rng(31)
    n, b = 640, 64
    sz = tile_sizes(n, b)
    q = len(sz)
    RA, RB = _rand_ranks(rng, q, b, True, 1, 12), _rand_ranks(rng, q, b, True, 1, 12)
    A, B = T.Shape(n, n, b, RA, True), T.Shape(n, n, b, RB, True)
    p = T.tlr_gemm_analyze("f64", "N", A, "N", B, ldc=n, flags=order | T.TLR_PLAN_VALIDATE)
    info = T.tlr_plan_info(p)
    L = [T.tlr_plan_launch(p, l) for l in range(info["launches"])]
    assert [x["stage"] for x in L] == [1, 4, 2, 3]
    if order == T.TLR_PLAN_FORCE_RIGHT:
        # X_i = D_A,ii W_{i,:} and the D_B,jj^T V_{:,j} blocks of T
        want = sum(2 * b * b * int(RB[i, :].sum()) for i in range(q)) + \
            sum(2 * b * b * int(RA[:, j].sum()) for j in range(q))
    else:
        # X'_j = V_{:,j}^T D_B,jj and the D_A,ii W_{i,:} blocks of Y
        want = sum(2 * b * b * int(RA[:, j].sum()) for j in range(q)) + \
            sum(2 * b * b * int(RB[i, :].sum()) for i in range(q))
    assert L[1]["useful_flops"] == want
    assert sum(x["useful_flops"] for x in L) == info["useful_flops"]
    # no diagonal: no side launch
    A0, B0 = T.Shape(n, n, b, RA, False), T.Shape(n, n, b, RB, False)
    p0 = T.tlr_gemm_analyze("f64", "N", A0, "N", B0, ldc=n, flags=order)
    assert [T.tlr_plan_launch(p0, l)["stage"] for l in range(T.tlr_plan_info(p0)["launches"])] == [1, 2, 3]


@pytest.mark.parametrize("seed", range(4))
def test_dense_a_plans(seed):
    # dense A x TLR B: the left order without a coupling stage; useful flops
    # equal the oracle's rank arithmetic exactly, and every plan (budgets,
    # streams, ops, ragged grids) passes the exhaustive descriptor check
    rng = np.random.default_rng(40 + seed)
    b = (16, 24, 32, 7)[seed]
    n = 5 * b - (0, 3, 0, 2)[seed]
    sz = tile_sizes(n, b)
    q = len(sz)
    diag = seed % 2 == 0
    RB = _rand_ranks(rng, q, b, diag, 0, min(b, 9))
    for r in range(q):
        for c in range(q):
            RB[r, c] = min(RB[r, c], sz[r], sz[c])
    B = T.Shape(n, n, b, RB, diag)
    for opA, opB in (("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")):
        m = n + 5
        dr, dc = (m, n) if opA == "N" else (n, m)
        p = T.tlr_gemm_analyze("f64", opA, None, opB, B, dr, dc, ldb=dr + 1, ldc=m, flags=T.TLR_PLAN_VALIDATE)
        info = T.tlr_plan_info(p)
        oB = pa.op_ranks(RB, opB)
        assert info["useful_flops"] == pa.useful_flops_dense_a(oB, sz, sz, m, diag)
        assert info["flops_right"] == -1 and info["final_flops_right"] == -1
        assert [T.tlr_plan_launch(p, l)["stage"] for l in range(info["launches"])] == [1, 3]
        assert all(T.tlr_plan_rect(p, r)["order"] == T.TLR_ORDER_LEFT for r in range(info["runs"]))
        full = info["workspace_bytes"]
        for frac, ns in ((0.3, 1), (0.3, 3), (1.0, 3)):
            try:
                p2 = T.tlr_gemm_analyze("f64", opA, None, opB, B, dr, dc, ldb=dr, ldc=m,
                                        workspace_budget=int(full * frac), n_streams=ns, flags=T.TLR_PLAN_VALIDATE)
            except T.TLRError as e:
                assert e.status == T.TLR_ERR_WORKSPACE
                continue
            i2 = T.tlr_plan_info(p2)
            assert i2["useful_flops"] == info["useful_flops"]
            assert i2["workspace_bytes"] <= max(int(full * frac), full if frac == 1.0 else 0)


def test_dense_a_errors():
    rng = np.random.default_rng(9)
    RB = _rand_ranks(rng, 3, 8, True, 0, 4)
    B = T.Shape(24, 24, 8, RB, True)
    with pytest.raises(T.TLRError) as e:
        T.tlr_gemm_analyze("f64", "N", None, "N", None, 10, 24, ldb=10, ldc=10)
    assert e.value.status == T.TLR_ERR_INVALID_ARG
    with pytest.raises(T.TLRError) as e:
        T.tlr_gemm_analyze("f64", "N", None, "N", B, 10, 23, ldb=10, ldc=10)      # k mismatch
    assert e.value.status == T.TLR_ERR_INVALID_ARG
    with pytest.raises(T.TLRError) as e:
        T.tlr_gemm_analyze("f64", "N", None, "N", B, 10, 24, ldb=9, ldc=10)       # lda < rows
    assert e.value.status == T.TLR_ERR_INVALID_ARG
    with pytest.raises(T.TLRError) as e:
        T.tlr_gemm_analyze("f64", "N", None, "N", B, 10, 24, ldb=10, ldc=10, flags=T.TLR_PLAN_FORCE_RIGHT)
    assert e.value.status == T.TLR_ERR_UNSUPPORTED


@pytest.mark.parametrize("seed", range(5))
def test_per_k_plans(seed):
    # the per-contraction-tile loop (comparator): its flop count equals the
    # brute-force tile loop's own multiply-add count, one rectangle (pass over
    # C) per contraction tile, and the exhaustive check passes (the first pass
    # writes C once, later passes each element at most once)
    from oracle import brute
    from tlr_inputs import random_tlr
    rng = np.random.default_rng(70 + seed)
    n, b = ((9, 3), (10, 4), (7, 2), (12, 5), (8, 4))[seed]
    diag = seed != 3
    A = random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
    B = random_tlr(rng, n, n, b, rank_lo=0, has_diag=diag, scale=1.0)
    for opA, opB in (("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")):
        sa, sb = T.Shape(n, n, b, A.ranks, diag), T.Shape(n, n, b, B.ranks, diag)
        p = T.tlr_gemm_analyze("f64", opA, sa, opB, sb, ldc=n + 1, flags=T.TLR_PLAN_PER_K | T.TLR_PLAN_VALIDATE)
        info = T.tlr_plan_info(p)
        _, flops = brute.tile_loop(1.0, opA, A, opB, B, 0.0, None, "right")
        assert info["useful_flops"] == flops
        assert info["runs"] == len(tile_sizes(n, b))
        stages = [T.tlr_plan_launch(p, l)["stage"] for l in range(info["launches"])]
        assert set(stages) <= {1, 2, 3} and stages.count(3) == info["runs"]
    with pytest.raises(T.TLRError) as e:
        T.tlr_gemm_analyze("f64", "N", sa, "N", None, n, n, ldb=n, ldc=n, flags=T.TLR_PLAN_PER_K)
    assert e.value.status == T.TLR_ERR_UNSUPPORTED


@pytest.mark.parametrize("flags", [T.TLR_PLAN_FORCE_LEFT, T.TLR_PLAN_FORCE_RIGHT, 0])
@pytest.mark.parametrize("which", ["A", "B"])
def test_no_coupling_plans_keep_stream_order(flags, which):
    """A rectangle with no coupling work (one operand block-diagonal: dense
    diagonal, every off-diagonal rank 0) still has diagonal-term products on
    the side stream.  Its fork event must be recorded on the group's stream
    before the side stream waits on it; the planner's own check of the
    enqueue order (run on every plan) rejects any other plan, so every
    analysis below must succeed, under budgets that split C into several
    rectangles, with and without boundary regions on their own streams."""
    rng = np.random.default_rng(31)
    for n, b, n_streams in ((256, 64, 1), (300, 64, 3)):
        q = -(-n // b)
        Z = np.zeros((q, q), np.int32)
        R = _rand_ranks(rng, q, b, True, 1, 20)
        sa = T.Shape(n, n, b, Z if which == "A" else R, True)
        sb = T.Shape(n, n, b, R if which == "A" else Z, True)
        for runs in (1, 2, 4):
            try:
                w = T.tlr_gemm_workspace_bytes("f64", "N", sa, "N", sb, n_streams=n_streams, flags=flags, runs=runs)
            except T.TLRError as e:           # the forced order cannot reach that many runs' budget
                assert e.status == T.TLR_ERR_WORKSPACE
                continue
            p = T.tlr_gemm_analyze("f64", "N", sa, "N", sb, ldc=n, workspace_budget=w, n_streams=n_streams,
                                   flags=flags | T.TLR_PLAN_VALIDATE)
            info = T.tlr_plan_info(p)
            stages = [T.tlr_plan_launch(p, l)["stage"] for l in range(info["launches"])]
            assert 1 not in stages
            assert 4 in stages

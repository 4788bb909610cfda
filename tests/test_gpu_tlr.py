"""TLR x TLR -> dense and TLR x dense -> dense on the GPU against the oracle,
on small seeded grids that span several 128 x 128 kernel blocks and ragged
tails: every op combination, beta in {0 (NaN-filled C), 0.5, 1}, both forced
association orders and the planner's own choice, rank-0 tiles, operands
without dense diagonals, boundary tiles (N not a multiple of b) with the
boundary regions on their own streams, workspace budgets that split C into
several rectangles, leading dimensions above the row count, fp64 and fp32,
and a grid large enough for the strip launch of the right/left product.
Bar: relative Frobenius error <= 1e-12 (fp64), <= 1e-5 (fp32)."""
import itertools

import numpy as np
import pytest

from gpu_helpers import TOL, check_tlr, gpu_ready, padded_tlr, run_tlr, say, transpose_tlr
from oracle import reference
from tlr_inputs import random_tlr

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ready(), reason="needs the GPU and libtlrgemm.so")]

F_RIGHT, F_LEFT = 0x1, 0x2


def _pair(seed, n, b, dtype="f64", lo=0, hi=24, diag=True, decay=1.0):
    rng = np.random.default_rng(seed)
    A = random_tlr(rng, n, n, b, rank_lo=lo, rank_hi=hi, has_diag=diag, dtype=dtype, decay=decay)
    B = random_tlr(rng, n, n, b, rank_lo=lo, rank_hi=hi, has_diag=diag, dtype=dtype, decay=decay)
    C = rng.standard_normal((n, n))
    return A, B, C


SHAPES = [(256, 64), (200, 64), (130, 32), (300, 128), (64, 64), (77, 16)]


@pytest.mark.parametrize("n,b", SHAPES)
@pytest.mark.parametrize("opA,opB", [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")])
def test_tlr_tlr_ops(n, b, opA, opB):
    for t, (beta, flags) in enumerate(itertools.product((0.0, 0.5, 1.0), (0, F_RIGHT, F_LEFT))):
        A, B, C = _pair(1000 * n + 7 * b + t, n, b)
        say(f"tlr n={n} b={b} {opA}{opB} beta={beta} flags={flags}")
        check_tlr(A, B, opA, opB, 0.75, beta, None if beta == 0 else C, flags=flags)


@pytest.mark.parametrize("n,b", [(256, 64), (130, 32), (300, 128)])
@pytest.mark.parametrize("opA,opB", [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")])
def test_tlr_dense_ops(n, b, opA, opB):
    rng = np.random.default_rng(n + b)
    A = random_tlr(rng, n, n, b, rank_lo=0, rank_hi=20, has_diag=True)
    for beta in (0.0, 0.5):
        ncols = n + 37
        Bd = rng.standard_normal((n, ncols) if opB == "N" else (ncols, n))
        C = rng.standard_normal((n, ncols))
        say(f"tlr x dense n={n} b={b} {opA}{opB} beta={beta}")
        check_tlr(A, Bd, opA, opB, 1.5, beta, None if beta == 0 else C, ld_pad=5)


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_no_diagonal_and_rank_zero(dtype):
    A, B, C = _pair(5, 250, 50, dtype=dtype, lo=0, hi=6, diag=False)
    A.ranks[1, 2] = 0
    A.U[(1, 2)] = A.U[(1, 2)][:, :0]
    A.V[(1, 2)] = A.V[(1, 2)][:, :0]
    for flags in (F_RIGHT, F_LEFT):
        say(f"no-diag {dtype} flags={flags}")
        check_tlr(A, B, "N", "N", 1.0, 0.5, C, flags=flags)


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("n_streams", [1, 3])
def test_budget_split_and_regions(dtype, n_streams):
    A, B, C = _pair(9, 600, 64, dtype=dtype, lo=2, hi=30)      # 10 x 10 tiles, last tile 24
    from hpc_linear_algebra_amd import tlrgemm as T
    sa = T.Shape(600, 600, 64, A.ranks, True)
    sb = T.Shape(600, 600, 64, B.ranks, True)
    for runs in (1, 3, 7):
        w = T.tlr_gemm_workspace_bytes(dtype, "N", sa, "N", sb, n_streams=n_streams, runs=runs)
        say(f"budget {dtype} streams={n_streams} runs<={runs} budget={w}")
        got, g = run_tlr(A, B, "N", "N", 1.0, 1.0, C, budget=w, n_streams=n_streams, return_plan=True)
        assert g.info["workspace_bytes"] <= w
        ref = reference.gemm_reference(1.0, "N", A, "N", B, 1.0, C)
        assert reference.rel_fro(got, ref) <= TOL[dtype]
        if n_streams > 1 and runs == 1:
            # enough workspace: the three boundary regions run beside the interior
            assert g.info["groups"] == 4
        assert g.info["groups"] in (1, 4)


def test_rank_zero_tiles_contribute_nothing():
    A, B, C = _pair(11, 256, 64, lo=1, hi=16)
    Az = padded_tlr(A, 0)
    for (i, j) in [(0, 1), (2, 3)]:
        Az.ranks[i, j] = 0
        Az.U[(i, j)] = Az.U[(i, j)][:, :0]
        Az.V[(i, j)] = Az.V[(i, j)][:, :0]
    for flags in (F_RIGHT, F_LEFT):
        got = run_tlr(Az, B, "N", "N", 1.0, 0.0, None, flags=flags)
        ref = reference.gemm_reference(1.0, "N", Az, "N", B, 0.0, None)
        assert reference.rel_fro(got, ref) <= 1e-12


def test_beta_zero_with_nan_and_inf_c():
    A, B, C = _pair(12, 200, 64)
    Cbad = np.full((200, 200), np.inf)
    Cbad[::3] = np.nan
    got = run_tlr(A, B, "N", "T", 1.0, 0.0, Cbad)
    ref = reference.gemm_reference(1.0, "N", A, "T", B, 0.0, None)
    assert np.all(np.isfinite(got)) and reference.rel_fro(got, ref) <= 1e-12


def test_uniform_rank_equals_padded():
    A, B, C = _pair(13, 256, 64, lo=3, hi=10)
    base = run_tlr(A, B, "N", "N", 1.0, 0.5, C)
    pad = run_tlr(padded_tlr(A, 10), padded_tlr(B, 10), "N", "N", 1.0, 0.5, C)
    ref = reference.gemm_reference(1.0, "N", A, "N", B, 0.5, C)
    assert reference.rel_fro(base, ref) <= 1e-12 and reference.rel_fro(pad, ref) <= 1e-12


@pytest.mark.parametrize("opA,opB", [("T", "N"), ("N", "T"), ("T", "T")])
def test_transpose_equals_swapped_factors(opA, opB):
    A, B, C = _pair(14, 200, 64)
    got = run_tlr(A, B, opA, opB, 0.5, 1.0, C)
    At = transpose_tlr(A) if opA == "T" else A
    Bt = transpose_tlr(B) if opB == "T" else B
    exp = run_tlr(At, Bt, "N", "N", 0.5, 1.0, C)
    assert reference.rel_fro(got, exp) <= 1e-12


def test_alpha_zero_scales_c():
    A, B, C = _pair(15, 130, 32)
    got = run_tlr(A, B, "N", "N", 0.0, -2.0, C)
    assert np.array_equal(got, -2.0 * C)


def test_empty_product():
    rng = np.random.default_rng(1)
    A = random_tlr(rng, 0, 0, 8, has_diag=True)
    got = run_tlr(A, A, "N", "N", 1.0, 0.0, None)
    assert got.shape == (0, 0)


def test_single_tile_and_full_rank():
    A, B, C = _pair(16, 100, 128)                           # q = 1: a dense GEMM
    check_tlr(A, B, "T", "N", 1.0, 0.5, C)
    A, B, C = _pair(17, 96, 32, lo=32, hi=32)               # every tile full rank
    check_tlr(A, B, "N", "N", 1.0, 0.5, C, flags=F_LEFT)


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_pipelined_rectangles_two_streams(dtype):
    # rectangles alternate between two arenas on two streams; the second stream
    # starts after the first rectangle's right product
    A, B, C = _pair(21, 700, 64, dtype=dtype, lo=1, hi=30)
    for budget in (0, 3_000_000):
        got, g = run_tlr(A, B, "T", "N", 1.0, 1.0, C, budget=budget, n_streams=2, flags=0x10,
                         return_plan=True)
        assert g.info["groups"] == 2 and g.info["runs"] >= 2
        ref = reference.gemm_reference(1.0, "T", A, "N", B, 1.0, C)
        assert reference.rel_fro(got, ref) <= TOL[dtype]


def _block_diagonal(t):
    """The operand with every off-diagonal tile dropped (rank 0): only the
    dense diagonal is left."""
    z = padded_tlr(t, 0)
    for key in list(z.U):
        z.ranks[key] = 0
        z.U[key] = z.U[key][:, :0]
        z.V[key] = z.V[key][:, :0]
    return z


@pytest.mark.parametrize("which", ["A", "B"])
@pytest.mark.parametrize("flags", [F_LEFT, F_RIGHT])
def test_no_coupling_back_to_back_executes(which, flags):
    """One operand block-diagonal (no coupling launch at all), a budget that
    splits C into several rectangles sharing one workspace arena, and two
    executes of one plan enqueued back to back with different values of the
    other operand.  The side launch of each rectangle writes its
    diagonal-term products into the arena; it must start only after the
    previous rectangle's (and the previous execute's) final update has read
    it.  Both results are compared with the oracle."""
    import torch
    from hpc_linear_algebra_amd import tlrgemm as T
    from hpc_linear_algebra_amd.device import DeviceTLR, TLRGemm, dense_from_device, dense_to_device
    n, b = 640, 64
    A1, B1, C = _pair(41, n, b, lo=4, hi=30)
    A2, B2, _ = _pair(42, n, b, lo=4, hi=30)
    if which == "A":
        A1 = _block_diagonal(A1)
        B2.ranks[:] = B1.ranks          # same structure, new values
        B2.U = {k: np.random.default_rng(7).standard_normal(v.shape) for k, v in B1.U.items()}
        B2.V = {k: np.random.default_rng(8).standard_normal(v.shape) for k, v in B1.V.items()}
        pairs = [(A1, B1), (A1, B2)]
    else:
        B1 = _block_diagonal(B1)
        A2.ranks[:] = A1.ranks
        A2.U = {k: np.random.default_rng(7).standard_normal(v.shape) for k, v in A1.U.items()}
        A2.V = {k: np.random.default_rng(8).standard_normal(v.shape) for k, v in A1.V.items()}
        pairs = [(A1, B1), (A2, B1)]
    dev = [(DeviceTLR(a), DeviceTLR(bb)) for a, bb in pairs]
    sa, sb = dev[0][0].shape, dev[0][1].shape
    w = T.tlr_gemm_workspace_bytes("f64", "N", sa, "N", sb, flags=flags, runs=4)
    g = TLRGemm("f64", "N", dev[0][0], "N", dev[0][1], ldc=n, budget=w, flags=flags)
    assert g.info["runs"] >= 2
    stages = [L["stage"] for L in g.launches()]
    assert 1 not in stages and 4 in stages
    Cs = [dense_to_device(C) for _ in pairs]
    say(f"no-coupling {which} flags={flags} runs={g.info['runs']} launches={len(stages)}")
    for (da, db), Cd in zip(dev, Cs):
        g(1.0, da, db, 0.5, Cd)
    torch.cuda.synchronize()
    for (a, bb), Cd in zip(pairs, Cs):
        got = dense_from_device(Cd, n, n)
        ref = reference.gemm_reference(1.0, "N", a, "N", bb, 0.5, C)
        assert reference.rel_fro(got, ref) <= 1e-12


@pytest.mark.parametrize("dtype,alpha", [("f32", 1e-29), ("f64", 1e-299)])
def test_tiny_alpha_large_c_does_not_overflow(dtype, alpha):
    """beta / alpha far above 1: C must not be pre-scaled by beta / alpha (that
    overflows for |C| ~ 1e10) but updated as alpha * sum + beta * C."""
    A, B, _ = _pair(51, 200, 64, dtype=dtype)
    C = 1e10 * np.random.default_rng(52).standard_normal((200, 200))
    check_tlr(A, B, "N", "N", alpha, 1.0, C)
    check_tlr(A, B, "T", "N", alpha, -0.5, C, flags=F_LEFT)


@pytest.mark.parametrize("dtype,opA,opB,flags,b", [("f64", "T", "N", F_LEFT, 128), ("f64", "N", "T", F_RIGHT, 128),
                                                   ("f32", "N", "N", F_LEFT, 128), ("f32", "T", "T", F_RIGHT, 128),
                                                   ("f64", "T", "N", F_LEFT, 129), ("f32", "N", "N", F_RIGHT, 129)])
def test_strip_launches(dtype, opA, opB, flags, b):
    """A 28 x 28 grid with ranks 0-20: the right or left product's tasks of
    rank <= 16 make enough 128 x 512 blocks for a strip launch, the others
    stay in the grouped launch; both against the oracle.  An odd tile size
    (b = 129: odd leading dimensions) puts the tasks in single-element load
    mode and gives every tile a one-row block."""
    n = 28 * b
    A, B, C = _pair(4200 + flags, n, b, dtype=dtype, lo=0, hi=20)
    say(f"strip launches {dtype} {opA}{opB} flags={flags} b={b}")
    check_tlr(A, B, opA, opB, 0.75, 0.5, C, flags=flags)
    got, g = run_tlr(A, B, opA, opB, 0.75, 0.5, C, flags=flags, return_plan=True)
    stage2 = [x for x in g.launches() if x["stage"] == 2]
    assert len(stage2) == 2 and min(x["tasks"] for x in stage2) > 0, stage2


@pytest.mark.parametrize("flags", [F_LEFT, F_RIGHT])
def test_strip_split_back_to_back_executes(flags):
    """Strip launches with the grouped right/left-product launch on the side
    stream, a budget that splits C into two rectangles sharing one workspace
    arena, and two executes of one plan enqueued back to back with different
    values of B.  Each rectangle's grouped launch must wait for its coupling
    (and so for the previous rectangle's and execute's final update), and the
    final update for it.  Both results against the oracle."""
    import torch
    from hpc_linear_algebra_amd import tlrgemm as T
    from hpc_linear_algebra_amd.device import DeviceTLR, TLRGemm, dense_from_device, dense_to_device
    n, b = 40 * 128, 128
    A, B1, C = _pair(4300 + flags, n, b, lo=0, hi=20)
    B2 = padded_tlr(B1, 0)               # same ranks, new values
    rng = np.random.default_rng(4400 + flags)
    B2.U = {k: rng.standard_normal(v.shape) / np.sqrt(b) for k, v in B1.U.items()}
    B2.V = {k: rng.standard_normal(v.shape) / np.sqrt(b) for k, v in B1.V.items()}
    dA, dB1, dB2 = DeviceTLR(A), DeviceTLR(B1), DeviceTLR(B2)
    w = T.tlr_gemm_workspace_bytes("f64", "N", dA.shape, "N", dB1.shape, flags=flags, runs=2)
    g = TLRGemm("f64", "N", dA, "N", dB1, ldc=n, budget=w, flags=flags)
    assert g.info["runs"] == 2
    assert sum(L["stage"] == 2 for L in g.launches()) == 4   # strip and grouped launch per rectangle
    Cs = [dense_to_device(C) for _ in range(2)]
    say(f"strip split back to back flags={flags}")
    for db, Cd in zip((dB1, dB2), Cs):
        g(1.0, dA, db, 0.5, Cd)
    torch.cuda.synchronize()
    for bb, Cd in zip((B1, B2), Cs):
        got = dense_from_device(Cd, n, n)
        ref = reference.gemm_reference(1.0, "N", A, "N", bb, 0.5, C)
        assert reference.rel_fro(got, ref) <= 1e-12

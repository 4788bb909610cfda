"""The 2u bar of the 16-bit parity tests, checked against the arithmetic it
was derived from.

The 16-bit path rounds the coupling blocks S, the right products T (or the
left products Y) and C to the 16-bit type once each, accumulating in float.
Emulated here in float64 with exactly those roundings (per tile, in the
order of "Tile-Low-Rank GEMM: Designing Storage Around the Contraction",
sections "One product, three stages" and "Association order and
workspace"), the relative Frobenius error against the oracle stays well
under 2u for both orders and both 16-bit types, while dropping a single
tile term exceeds it."""
import numpy as np
import pytest
import torch

from oracle import reference
from tlr_inputs import on_grid, random_tlr

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _round(x, dt):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return t.to(torch.float16 if dt == "f16" else torch.bfloat16).to(torch.float64).numpy()


def _emulate(A, B, alpha, beta, C, dt, order, drop=None):
    rs, ks, cs = A.row_sizes, A.col_sizes, B.col_sizes
    ro, co = reference.offsets(rs), reference.offsets(cs)
    out = beta * np.asarray(C, dtype=np.float64)
    f64 = lambda x: np.asarray(x, dtype=np.float64)
    for i in range(len(rs)):
        for j in range(len(cs)):
            acc = np.zeros((rs[i], cs[j]))
            for k in range(len(ks)):
                if drop == (i, k, j):
                    continue
                da, db = A.has_diag and i == k, B.has_diag and k == j
                if da and db:
                    acc += f64(A.diag[i]) @ f64(B.diag[k])
                elif da:
                    if B.ranks[k, j]:
                        acc += _round(f64(A.diag[i]) @ f64(B.U[(k, j)]), dt) @ f64(B.V[(k, j)]).T
                elif db:
                    if A.ranks[i, k]:
                        acc += f64(A.U[(i, k)]) @ _round(f64(A.V[(i, k)]).T @ f64(B.diag[k]), dt)
                elif A.ranks[i, k] and B.ranks[k, j]:
                    S = _round(f64(A.V[(i, k)]).T @ f64(B.U[(k, j)]), dt)
                    if order == "right":
                        acc += f64(A.U[(i, k)]) @ _round(S @ f64(B.V[(k, j)]).T, dt)
                    else:
                        acc += _round(f64(A.U[(i, k)]) @ S, dt) @ f64(B.V[(k, j)]).T
            out[ro[i]:ro[i] + rs[i], co[j]:co[j] + cs[j]] += alpha * acc
    return _round(out, dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("order", ["right", "left"])
def test_emulated_rounding_stays_under_the_bar(dt, order):
    rng = np.random.default_rng(8 if dt == "f16" else 9)
    A = random_tlr(rng, 256, 256, 32, 4, 24, has_diag=True, dtype=dt)
    B = random_tlr(rng, 256, 256, 32, 4, 24, has_diag=True, dtype=dt)
    C = on_grid(rng.standard_normal((256, 256)), dt)
    for beta, Cin in ((0.0, None), (1.0, C)):
        ref = reference.gemm_reference(1.0, "N", A, "N", B, beta, Cin)
        got = _emulate(A, B, 1.0, beta, np.zeros((256, 256)) if Cin is None else Cin, dt, order)
        err = reference.rel_fro(got, ref)
        assert err <= 1.0 * U[dt], (beta, err / U[dt])     # measured 0.4u - 0.8u; the bar is 2u


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_a_dropped_tile_term_exceeds_the_bar(dt):
    rng = np.random.default_rng(10)
    A = random_tlr(rng, 256, 256, 64, 16, 32, has_diag=True, dtype=dt)
    B = random_tlr(rng, 256, 256, 64, 16, 32, has_diag=True, dtype=dt)
    ref = reference.gemm_reference(1.0, "N", A, "N", B, 0.0, None)
    got = _emulate(A, B, 1.0, 0.0, np.zeros((256, 256)), dt, "left", drop=(1, 2, 3))
    assert reference.rel_fro(got, ref) > 2.0 * U[dt]


def _bound_parts(A, B, beta, C):
    from gpu_helpers import abs_operand
    scale = reference.gemm_reference(1.0, "N", abs_operand(A), "N", abs_operand(B), abs(beta),
                                     None if beta == 0 else np.abs(np.asarray(C, np.float64)))
    return scale


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("order", ["right", "left"])
def test_emulated_rounding_within_the_element_bound(dt, order):
    """The per-element bound of the GPU tests (gpu_helpers.check_elements)
    holds for every element of the emulated 16-bit arithmetic, and one
    element moved by a tenth of the largest entry breaks it."""
    from gpu_helpers import check_elements
    rng = np.random.default_rng(12)
    A = random_tlr(rng, 192, 192, 32, 4, 24, has_diag=True, dtype=dt)
    B = random_tlr(rng, 192, 192, 32, 4, 24, has_diag=True, dtype=dt)
    C = on_grid(rng.standard_normal((192, 192)), dt)
    ref = reference.gemm_reference(1.0, "N", A, "N", B, 1.0, C)
    got = _emulate(A, B, 1.0, 1.0, C, dt, order)
    scale = _bound_parts(A, B, 1.0, C)
    check_elements(got, ref, scale, dt, 192, 32)
    bad = got.copy()
    bad[37, 101] += 0.1 * np.max(np.abs(ref))
    with pytest.raises(AssertionError):
        check_elements(bad, ref, scale, dt, 192, 32)


@pytest.mark.parametrize("order", ["right", "left"])
def test_float32_arithmetic_within_the_element_bound(order):
    """The same for float32: the three stages evaluated tile by tile in numpy
    float32 (every product and stored intermediate rounded to float32) stay
    within the fp32 element bound; a wrong element of a tenth of the largest
    entry does not."""
    from gpu_helpers import check_elements
    rng = np.random.default_rng(13)
    A = random_tlr(rng, 200, 200, 48, 2, 30, has_diag=True, dtype="f32")
    B = random_tlr(rng, 200, 200, 48, 2, 30, has_diag=True, dtype="f32")
    C = rng.standard_normal((200, 200)).astype(np.float32)
    rs = A.row_sizes
    off = reference.offsets(rs)
    got = np.zeros((200, 200), np.float32)
    for i in range(len(rs)):
        for j in range(len(rs)):
            acc = np.zeros((rs[i], rs[j]), np.float32)
            for k in range(len(rs)):
                da, db = i == k, k == j
                if da and db:
                    acc += A.diag[i] @ B.diag[k]
                elif da:
                    acc += (A.diag[i] @ B.U[(k, j)]) @ B.V[(k, j)].T
                elif db:
                    acc += A.U[(i, k)] @ (A.V[(i, k)].T @ B.diag[k])
                else:
                    S = A.V[(i, k)].T @ B.U[(k, j)]
                    acc += A.U[(i, k)] @ (S @ B.V[(k, j)].T) if order == "right" else (A.U[(i, k)] @ S) @ B.V[(k, j)].T
            got[off[i]:off[i] + rs[i], off[j]:off[j] + rs[j]] = np.float32(0.5) * acc + np.float32(0.75) * \
                C[off[i]:off[i] + rs[i], off[j]:off[j] + rs[j]]
    ref = reference.gemm_reference(0.5, "N", A, "N", B, 0.75, C)
    from gpu_helpers import abs_operand
    scale = reference.gemm_reference(0.5, "N", abs_operand(A), "N", abs_operand(B), 0.75, np.abs(C.astype(np.float64)))
    check_elements(got, ref, scale, "f32", 200, 48)
    bad = got.copy()
    bad[5, 190] += np.float32(0.1 * np.max(np.abs(ref)))
    with pytest.raises(AssertionError):
        check_elements(bad, ref, scale, "f32", 200, 48)

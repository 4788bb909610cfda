"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the oracle.  (Not collected by pytest: no test_ prefix.)"""
from __future__ import annotations

import copy
import sys

import numpy as np

from oracle import reference
from tlr_inputs import TLRTiles

# fp64 / fp32: the stated bars.  16-bit types: 2u, u the unit roundoff (2^-11
# half, 2^-8 bfloat16).  The 16-bit path rounds the coupling blocks, the right
# or left products and C once each; a rounding is a relative error of at most
# u, about u/sqrt(3) RMS, and for inputs with independent signs the three add
# in quadrature to about u in relative Frobenius norm (an emulation in float64
# of exactly those roundings measured 0.43u-0.74u on the test shapes).  The
# float accumulation adds at most K * 2^-24 per element, far below u.
TOL = {"f64": 1e-12, "f32": 1e-5, "f16": 2.0 * 2.0 ** -11, "bf16": 2.0 * 2.0 ** -8}

# unit roundoff of each element type; 16-bit products accumulate in float
UNIT = {"f64": 2.0 ** -53, "f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
ACC_UNIT = {"f64": 2.0 ** -53, "f32": 2.0 ** -24, "f16": 2.0 ** -24, "bf16": 2.0 ** -24}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_ready():
    try:
        import torch
        if not torch.cuda.is_available():
            return False
        from hpc_linear_algebra_amd import tlrgemm
        tlrgemm.lib()
        return True
    except Exception:
        return False


def op_dims(t, op):
    return (t.rows, t.cols) if op == "N" else (t.cols, t.rows)


def run_tlr(A, B, opA: str, opB: str, alpha: float, beta: float, C_in,
            budget: int = 0, n_streams: int = 1, flags: int = 0, ld_pad: int = 0, return_plan=False,
            dtype: str = None):
    """C = alpha op(A) op(B) + beta C_in on the GPU; C_in None -> NaN-filled C.
    Either A or B may be a dense array (the other a TLRTiles)."""
    import torch
    from hpc_linear_algebra_amd.device import DeviceTLR, TLRGemm, dense_from_device, dense_to_device
    dense_a = not isinstance(A, TLRTiles)
    dense = not isinstance(B, TLRTiles)
    dtype = dtype or (B.dtype if dense_a else A.dtype)
    npd = np.float64 if dtype == "f64" else np.float32   # 16-bit values travel in float32 arrays
    if dense_a:
        m = A.shape[0] if opA == "N" else A.shape[1]
    else:
        m = op_dims(A, opA)[0]
    if dense:
        n = B.shape[1] if opB == "N" else B.shape[0]
    else:
        n = op_dims(B, opB)[1]
    ldc = max(1, m + ld_pad)
    Cstart = np.full((m, n), np.nan, dtype=npd) if C_in is None else np.asarray(C_in, dtype=npd)
    if dense_a:
        lda = max(1, A.shape[0] + ld_pad)
        dA = dense_to_device(np.asarray(A, dtype=npd), ld=lda, dtype=dtype)
        dB = DeviceTLR(B)
        g = TLRGemm(dtype, opA, None, opB, dB, ldc=ldc, dense_shape=A.shape, ldb=lda, budget=budget,
                    n_streams=n_streams, flags=flags)
    elif dense:
        dA = DeviceTLR(A)
        ldb = max(1, B.shape[0] + ld_pad)
        dB = dense_to_device(np.asarray(B, dtype=npd), ld=ldb, dtype=dtype)
        g = TLRGemm(dtype, opA, dA, opB, None, ldc=ldc, dense_shape=B.shape, ldb=ldb, budget=budget,
                    n_streams=n_streams, flags=flags)
    else:
        dA = DeviceTLR(A)
        dB = DeviceTLR(B)
        g = TLRGemm(dtype, opA, dA, opB, dB, ldc=ldc, budget=budget, n_streams=n_streams, flags=flags)
    Cd = dense_to_device(Cstart, ld=ldc, dtype=dtype)
    side = [torch.cuda.Stream() for _ in range(n_streams - 1)]
    streams = [torch.cuda.current_stream().cuda_stream] + [s.cuda_stream for s in side]
    g(alpha, dA, dB, beta, Cd, streams)
    torch.cuda.synchronize()
    out = dense_from_device(Cd, m, n)
    if return_plan:
        return out, g
    return out


def abs_operand(t):
    """The operand with every factor, diagonal tile or dense entry replaced by
    its absolute value (rebuilt, tile (i,j) is |U_ij| |V_ij|^T)."""
    if not isinstance(t, TLRTiles):
        return np.abs(np.asarray(t, dtype=np.float64))
    a = copy.copy(t)
    a.U = {k: np.abs(np.asarray(v, dtype=np.float64)) for k, v in t.U.items()}
    a.V = {k: np.abs(np.asarray(v, dtype=np.float64)) for k, v in t.V.items()}
    a.diag = None if t.diag is None else [np.abs(np.asarray(d, dtype=np.float64)) for d in t.diag]
    return a


def element_bound_factor(dtype: str, k: int, b: int) -> float:
    """Factor f of the per-element bound |C_gpu - C| <= f * scale, scale =
    |alpha| |A|_f |B|_f + |beta| |C_in| with |X|_f the operand rebuilt from
    the absolute values of its factors.  Every element is an inner product
    along a chain of at most three products: the coupling (inner length
    <= b), the right or left product (<= b) and the final update (<= k + b
    with the diagonal-term segment), so the first-order rounding bound of a
    product chain gives (k + 3b) accumulation roundings plus the roundings of
    the stored intermediates and of alpha / beta.  For the 16-bit types the
    three stored results (coupling, right/left product, C) are rounded to the
    16-bit type and the sums are accumulated in float.  fp64 is compared with
    an fp64 oracle whose own error obeys the same bound: factor 2."""
    acc = (k + 3 * b + 4) * ACC_UNIT[dtype]
    if dtype in ("f16", "bf16"):
        return 3 * UNIT[dtype] + acc
    return 2 * acc if dtype == "f64" else acc


def check_elements(got, ref, scale, dtype: str, k: int, b: int, what: str = ""):
    """Per-element bound of element_bound_factor (catches one wrong block or
    element that a norm over the whole matrix would hide)."""
    f = element_bound_factor(dtype, k, b)
    bad = np.abs(np.asarray(got, np.float64) - ref) > f * scale + 1e-300
    if np.any(bad):
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what} {int(bad.sum())} elements beyond the per-element bound, e.g. ({r},{c}): "
                             f"got {got[r, c]!r} ref {ref[r, c]!r} bound {f * scale[r, c]:.3e}")


def inner_dim(A, opA):
    if isinstance(A, TLRTiles):
        return op_dims(A, opA)[1]
    A = np.asarray(A)
    return A.shape[1] if opA == "N" else A.shape[0]


def check_tlr(A, B, opA, opB, alpha, beta, C_in, **kw):
    """The GPU product against the oracle: relative Frobenius error within
    TOL and every element within the per-element bound."""
    got = run_tlr(A, B, opA, opB, alpha, beta, C_in, **kw)
    ref = reference.gemm_reference(alpha, opA, A, opB, B, beta, C_in)
    err = reference.rel_fro(got, ref)
    dtype = kw.get("dtype") or (A.dtype if isinstance(A, TLRTiles) else B.dtype)
    assert np.all(np.isfinite(got)), "non-finite output"
    assert err <= TOL[dtype], f"relative Frobenius error {err:.3e} > {TOL[dtype]:.0e}"
    scale = reference.gemm_reference(abs(alpha), opA, abs_operand(A), opB, abs_operand(B), abs(beta),
                                     None if beta == 0 else np.abs(np.asarray(C_in, np.float64)))
    tb = A.b if isinstance(A, TLRTiles) else B.b
    check_elements(got, ref, scale, dtype, inner_dim(A, opA), tb)
    return err


def transpose_tlr(t: TLRTiles) -> TLRTiles:
    U = {(j, i): t.V[(i, j)].copy() for (i, j) in t.U}
    V = {(j, i): t.U[(i, j)].copy() for (i, j) in t.U}
    D = None if t.diag is None else [d.T.copy() for d in t.diag]
    return TLRTiles(t.cols, t.rows, t.b, t.ranks.T.copy(), D, U, V, t.dtype)


def padded_tlr(t: TLRTiles, rmax: int) -> TLRTiles:
    p = copy.deepcopy(t)
    for key in list(p.U):
        u, v = p.U[key], p.V[key]
        r = u.shape[1]
        want = min(rmax, u.shape[0], v.shape[0])
        if want > r:
            p.U[key] = np.concatenate([u, np.zeros((u.shape[0], want - r), u.dtype)], axis=1)
            p.V[key] = np.concatenate([v, np.zeros((v.shape[0], want - r), v.dtype)], axis=1)
            p.ranks[key] = want
    return p

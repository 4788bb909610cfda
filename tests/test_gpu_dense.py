"""The MFMA GEMM kernel on dense matrices (tlr_dense_gemm) against float64
numpy, through the C ABI: every op combination, ragged edges (including the
2053 x 2039 x 2048 shape the tiled-GEMM page tests), leading dimensions above
the row count, fp32, beta = 0 with a NaN-filled C, alpha = 0, k = 0."""
import numpy as np
import pytest

from gpu_helpers import gpu_ready, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ready(), reason="needs the GPU and libtlrgemm.so")]


def _run(dtype, opA, opB, m, n, k, alpha, beta, seed=0, pad=0, nan_c=False):
    import torch
    from hpc_linear_algebra_amd import tlrgemm as T
    from hpc_linear_algebra_amd.device import dense_from_device, dense_to_device
    say(f"dense {dtype} {opA}{opB} m={m} n={n} k={k} alpha={alpha} beta={beta}")
    rng = np.random.default_rng(seed)
    npd = np.float64 if dtype == "f64" else np.float32
    Ash = (m, k) if opA == "N" else (k, m)
    Bsh = (k, n) if opB == "N" else (n, k)
    A = rng.standard_normal(Ash).astype(npd)
    B = rng.standard_normal(Bsh).astype(npd)
    C = np.full((m, n), np.nan, npd) if nan_c else rng.standard_normal((m, n)).astype(npd)
    lda, ldb, ldc = Ash[0] + pad, Bsh[0] + pad, m + pad
    dA, dB, dC = dense_to_device(A, ld=max(1, lda)), dense_to_device(B, ld=max(1, ldb)), dense_to_device(C, ld=max(1, ldc))
    T.tlr_dense_gemm(dtype, opA, opB, m, n, k, alpha, dA.data_ptr(), max(1, lda), dB.data_ptr(), max(1, ldb),
                     beta, dC.data_ptr(), max(1, ldc), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = dense_from_device(dC, m, n)
    Ad = A.astype(np.float64) if opA == "N" else A.astype(np.float64).T
    Bd = B.astype(np.float64) if opB == "N" else B.astype(np.float64).T
    ref = alpha * (Ad @ Bd)
    if beta != 0:
        ref = ref + beta * C.astype(np.float64)
    assert np.all(np.isfinite(got))
    den = max(np.linalg.norm(ref), 1e-300)
    err = np.linalg.norm(got - ref) / den
    tol = 1e-13 if dtype == "f64" else 2e-6
    assert err <= tol, err
    # per-element check as well: catches a wrong block that a norm could hide
    scale = np.abs(Ad) @ np.abs(Bd) * abs(alpha) + (abs(beta) * np.abs(C) if beta != 0 else 0)
    assert np.all(np.abs(got - ref) <= 64 * np.finfo(npd).eps * (scale + 1e-300) + 1e-300)


@pytest.mark.parametrize("opA,opB", [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_ops_ragged(opA, opB, dtype):
    _run(dtype, opA, opB, 300, 257, 131, 1.25, 0.5, seed=1, pad=3)


def test_tiled_gemm_page_shape():
    _run("f64", "N", "N", 2053, 2039, 2048, 1.0, 0.0, seed=2)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (128, 128, 16), (129, 1, 17), (5, 300, 3), (64, 64, 1000)])
def test_small_shapes(m, n, k):
    _run("f64", "N", "N", m, n, k, -0.5, 2.0, seed=3)


def test_beta_zero_ignores_nan_c():
    _run("f64", "N", "T", 200, 190, 70, 1.0, 0.0, seed=4, nan_c=True)
    _run("f32", "T", "N", 200, 190, 70, 1.0, 0.0, seed=4, nan_c=True)


def test_alpha_zero_and_k_zero():
    _run("f64", "N", "N", 100, 90, 40, 0.0, 0.75, seed=5)
    _run("f64", "N", "N", 100, 90, 0, 1.0, 0.75, seed=6)


def test_square_fp64_large():
    _run("f64", "T", "N", 1536, 1536, 1536, 1.0, 1.0, seed=7)

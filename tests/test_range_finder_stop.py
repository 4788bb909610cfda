"""The early stop of the randomized range finder on the host: the rule the
QR of the sketches applies (after every fourth column, at least 8 samples
left, stop once the sketch's remaining energy E satisfies
E <= 1e-10 tol^2 (s - k) ||X||_F^2), emulated with numpy on tiles of the
TLR-output recipe at a reduced size.  It checks the reading the GPU path
relies on: at the stop, the energy the basis leaves out of X is far below
1e-7 tol^2 ||X||_F^2, so the truncation ranks are those of the full sketch,
and the recipe's tiles do stop short of the full sketch width.  No kernel is
launched."""
import numpy as np

from oracle import reference
from oracle import recompress
from tlr_inputs.gen import TLR_OUT, tlr_out_inputs

STOP = 1e-10     # the stop constant of the range finder
SAMPLES = 8      # samples beyond max_rank (the oracle's sketch width is max_rank + 8)


def _stop_point(Y, nx, tol):
    s = Y.shape[1]
    for k in range(4, s - SAMPLES + 1, 4):
        Qk, _ = np.linalg.qr(Y[:, :k])
        E = float(np.sum((Y[:, k:] - Qk @ (Qk.T @ Y[:, k:])) ** 2))
        if E <= STOP * tol * tol * (s - k) * nx:
            return k
    return s


def test_stop_leaves_out_negligible_energy_and_keeps_the_ranks():
    N, b = 1024, 256
    A, B, C, omega = tlr_out_inputs(N=N, b=b)
    tol = TLR_OUT["tol"]
    X = reference.gemm_reference(1.0, "N", A, "N", B, 1.0, reference.reconstruct(C))
    q = N // b
    stops = []
    for i in range(q):
        for j in range(q):
            if i == j:
                continue
            Xt = X[i * b:(i + 1) * b, j * b:(j + 1) * b]
            nx = float(np.sum(Xt * Xt))
            Y = Xt @ omega
            k = _stop_point(Y, nx, tol)
            stops.append(k)
            Qk, _ = np.linalg.qr(Y[:, :k])
            left = float(np.sum((Xt - Qk @ (Qk.T @ Xt)) ** 2))
            assert left <= 1e-7 * tol * tol * nx, (i, j, k, left / (tol * tol * nx))
            # the truncation of the projected tile keeps the rank of the exact one
            Qs, _ = np.linalg.qr(Y)
            r_full = recompress.truncation_rank(np.linalg.svd(Qs.T @ Xt, compute_uv=False),
                                                float(np.sqrt(nx)), tol)
            r_stop = recompress.truncation_rank(np.linalg.svd(Qk.T @ Xt, compute_uv=False),
                                                float(np.sqrt(nx)), tol)
            assert r_stop == r_full, (i, j, r_stop, r_full)
    assert max(stops) < omega.shape[1]          # every tile stopped early

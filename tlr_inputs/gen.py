"""Seeded generators for TLR operands, dense matrices and the five workloads.

A TLR operand is kept here *per tile*: a rank table, a list of dense diagonal
tiles, and one (U_ij, V_ij) factor pair per off-diagonal tile, following the
storage model of "TLR Matrix Multiplication" (section "Introduction: TLR GEMM":
dense diagonal tiles, off-diagonal tiles U_ij V_ij^T of rank r_ij, smaller
boundary tiles when N is not a multiple of b).  Packing into the library's
buffers is done elsewhere; the oracle reads these per-tile arrays directly.

Seeds: ``numpy.random.default_rng(1000*c + stream)`` for workload c, with
stream 0 = ranks of A, 1 = ranks of B, 2 = values of A, 3 = values of B (or the
dense B), 4 = the input C.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np


def tile_sizes(n: int, b: int) -> List[int]:
    """Tile extents along one dimension: b, ..., b, then the remainder."""
    if n <= 0:
        return []
    q = -(-n // b)
    sizes = [b] * q
    rem = n - (q - 1) * b
    sizes[-1] = rem
    return sizes


@dataclass
class TLRTiles:
    """One TLR matrix stored tile by tile.

    ``ranks[i, j]`` is the rank of tile (i, j); ``U[(i, j)]`` has shape
    (row_sizes[i], r) and ``V[(i, j)]`` shape (col_sizes[j], r), so the tile
    equals U @ V.T.  ``diag[i]`` holds the dense tile (i, i) when the operand
    has a dense diagonal; ranks[i, i] is then 0.  Values are float64 or
    float32 numpy arrays (``dtype`` 'f64' / 'f32'; for 'f16' / 'bf16' float32
    arrays whose values are on the 16-bit type's grid).
    """
    rows: int
    cols: int
    b: int
    ranks: np.ndarray
    diag: Optional[List[np.ndarray]]
    U: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)
    V: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)
    dtype: str = "f64"

    @property
    def row_sizes(self) -> List[int]:
        return tile_sizes(self.rows, self.b)

    @property
    def col_sizes(self) -> List[int]:
        return tile_sizes(self.cols, self.b)

    @property
    def qr(self) -> int:
        return len(self.row_sizes)

    @property
    def qc(self) -> int:
        return len(self.col_sizes)

    @property
    def has_diag(self) -> bool:
        return self.diag is not None


def _np_dtype(dtype: str):
    """Host array type of an element type: 16-bit values are held in float32
    arrays (numpy has no bfloat16), each value on the 16-bit type's grid."""
    return {"f64": np.float64, "f32": np.float32, "f16": np.float32, "bf16": np.float32}[dtype]


def on_grid(x: np.ndarray, dtype: str) -> np.ndarray:
    """x in the host array type of ``dtype``, rounded to nearest-even onto that
    type's values (for 16-bit types: half, or bfloat16 = the upper 16 bits of a
    float32).  Input preparation only: drawn values become representable."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return f
    if dtype == "f16":
        return f.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = f.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32).reshape(f.shape)
    raise ValueError(dtype)


def ranks_from_fn(qr: int, qc: int, fn: Callable[[int, int], int],
                  has_diag: bool = True) -> np.ndarray:
    """Rank table with r[i, j] = fn(i, j) off the diagonal (0 on it if dense)."""
    R = np.zeros((qr, qc), dtype=np.int32)
    for i in range(qr):
        for j in range(qc):
            if has_diag and i == j:
                continue
            R[i, j] = fn(i, j)
    return R


def fill_values(rng: np.random.Generator, rows: int, cols: int, b: int,
                ranks: np.ndarray, has_diag: bool, dtype: str = "f64",
                decay: float = 1.0, scale: Optional[float] = None) -> TLRTiles:
    """Draw N(0,1)*scale entries: diagonal tiles first, then factor pairs in
    tile-row-major order (U before V), then scale rank column a by decay**a."""
    rs, cs = tile_sizes(rows, b), tile_sizes(cols, b)
    if scale is None:
        scale = 1.0 / math.sqrt(b)
    diag = None
    if has_diag:
        assert rows == cols
        diag = [rng.standard_normal((s, s)) * scale for s in rs]
    U, V = {}, {}
    for i in range(len(rs)):
        for j in range(len(cs)):
            if has_diag and i == j:
                continue
            r = int(ranks[i, j])
            u = rng.standard_normal((rs[i], r)) * scale
            v = rng.standard_normal((cs[j], r)) * scale
            if decay != 1.0 and r > 0:
                w = decay ** np.arange(r)
                u = u * w
                v = v * w
            U[(i, j)] = u
            V[(i, j)] = v
    if dtype != "f64":
        diag = None if diag is None else [on_grid(d, dtype) for d in diag]
        U = {k: on_grid(x, dtype) for k, x in U.items()}
        V = {k: on_grid(x, dtype) for k, x in V.items()}
    return TLRTiles(rows, cols, b, ranks.astype(np.int32), diag, U, V, dtype)


def random_tlr(rng: np.random.Generator, rows: int, cols: int, b: int,
               rank_lo: int = 0, rank_hi: Optional[int] = None,
               has_diag: Optional[bool] = None, dtype: str = "f64",
               decay: float = 1.0, scale: Optional[float] = None) -> TLRTiles:
    """Random TLR operand with off-diagonal ranks uniform in [rank_lo, rank_hi]
    (clipped to each tile's smaller side)."""
    rs, cs = tile_sizes(rows, b), tile_sizes(cols, b)
    if has_diag is None:
        has_diag = rows == cols
    R = np.zeros((len(rs), len(cs)), dtype=np.int32)
    for i in range(len(rs)):
        for j in range(len(cs)):
            if has_diag and i == j:
                continue
            hi = min(rs[i], cs[j]) if rank_hi is None else min(rank_hi, rs[i], cs[j])
            lo = min(rank_lo, hi)
            R[i, j] = rng.integers(lo, hi + 1)
    return fill_values(rng, rows, cols, b, R, has_diag, dtype, decay, scale)


def basis_tlr(rng: np.random.Generator, rows: int, cols: int, b: int, r0: int, rank_lo: int, rank_hi: int,
              shared: str, has_diag: bool = True, decay: float = 1.0, dtype: str = "f64") -> TLRTiles:
    """TLR operand whose factors are drawn inside shared bases, so that
    products of such operands have tiles of bounded rank (the compressible
    outputs a TLR-output product is for).  Draw order: the diagonal tiles,
    then one basis per tile row (s_i x r0) when the outer factors are shared,
    one per tile column (s_j x r0) when the inner ones are, then per
    off-diagonal tile (tile-row-major) its rank and its coefficient or free
    factors.  Entries N(0,1)/sqrt(b); basis column a scaled by decay**a;
    coefficients N(0,1)/sqrt(r0).  A shared outer factor of tile (i,j) is
    Phi_i G_ij (G_ij r0 x r_ij), a shared inner one Psi_j H_ij; ``shared`` is
    "outer", "inner" or "both"."""
    rs, cs = tile_sizes(rows, b), tile_sizes(cols, b)
    scale = 1.0 / math.sqrt(b)
    diag = [rng.standard_normal((s_, s_)) * scale for s_ in rs] if has_diag else None
    w = decay ** np.arange(r0)
    phi = [rng.standard_normal((s_, r0)) * scale * w for s_ in rs] if shared in ("outer", "both") else None
    psi = [rng.standard_normal((s_, r0)) * scale * w for s_ in cs] if shared in ("inner", "both") else None
    R = np.zeros((len(rs), len(cs)), dtype=np.int32)
    U, V = {}, {}
    for i in range(len(rs)):
        for j in range(len(cs)):
            if has_diag and i == j:
                continue
            r = int(rng.integers(min(rank_lo, rs[i], cs[j]), min(rank_hi, rs[i], cs[j]) + 1))
            R[i, j] = r
            u = phi[i] @ (rng.standard_normal((r0, r)) / math.sqrt(r0)) if phi is not None \
                else rng.standard_normal((rs[i], r)) * scale
            v = psi[j] @ (rng.standard_normal((r0, r)) / math.sqrt(r0)) if psi is not None \
                else rng.standard_normal((cs[j], r)) * scale
            U[(i, j)], V[(i, j)] = u, v
    if dtype != "f64":
        diag = None if diag is None else [on_grid(d, dtype) for d in diag]
        U = {k: on_grid(x, dtype) for k, x in U.items()}
        V = {k: on_grid(x, dtype) for k, x in V.items()}
    return TLRTiles(rows, cols, b, R, diag, U, V, dtype)


def gaussian_sketch(seed: int, b: int, s: int, dtype: str = "f64") -> np.ndarray:
    """b x s matrix of N(0,1) entries (the range sketch of dense-to-TLR
    compression), from numpy.random.default_rng(seed)."""
    return on_grid(np.random.default_rng(seed).standard_normal((b, s)), dtype)


# The TLR-output product (C <- alpha A B + beta C with C in TLR format,
# compressed to a tolerance): A's outer factors share one basis per tile row,
# B's inner factors one per tile column, C both, so every result tile has
# rank at most r0 plus the ranks of the diagonal-term products.
TLR_OUT = dict(name="tlr_out_f64_n8192_b256", kind="tlr_out", dtype="f64", N=8192, b=256, opA="N", opB="N",
               alpha=1.0, beta=1.0, r0=16, rank_lo=4, rank_hi=12, c_rank_lo=0, c_rank_hi=8, decay=0.5,
               tol=1e-6, max_rank=48, seed=6000)


def tlr_out_inputs(cfg: Optional[dict] = None, N: Optional[int] = None, b: Optional[int] = None,
                   dtype: Optional[str] = None):
    """(A, B, C, omega) of a TLR-output product: the TLR_OUT workload, or the
    same recipe at another size.  Seeds 1000*6 + stream: 0 = A, 1 = B, 2 = C,
    3 = the sketch."""
    cfg = dict(TLR_OUT if cfg is None else cfg)
    N = N or cfg["N"]
    b = b or cfg["b"]
    dt = dtype or cfg["dtype"]
    sd = cfg["seed"]
    A = basis_tlr(np.random.default_rng(sd + 0), N, N, b, cfg["r0"], cfg["rank_lo"], cfg["rank_hi"], "outer",
                  True, cfg["decay"], dt)
    B = basis_tlr(np.random.default_rng(sd + 1), N, N, b, cfg["r0"], cfg["rank_lo"], cfg["rank_hi"], "inner",
                  True, cfg["decay"], dt)
    C = basis_tlr(np.random.default_rng(sd + 2), N, N, b, cfg["r0"], cfg["c_rank_lo"], cfg["c_rank_hi"], "both",
                  True, cfg["decay"], dt)
    omega = gaussian_sketch(sd + 3, b, cfg["max_rank"] + 8, dt)
    return A, B, C, omega


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------
CONFIGS = {
    1: dict(name="tlr_tlr_f64_n512_b64", kind="tlr_tlr", dtype="f64", N=512, b=64,
            opA="N", opB="N", alpha=1.0, beta=0.0, budget=None, decay=1.0),
    2: dict(name="tlr_dense_f64_n4096_b256", kind="tlr_dense", dtype="f64", N=4096, b=256,
            opA="N", opB="N", alpha=1.5, beta=0.5, budget=None, decay=0.8),
    3: dict(name="tlr_tlr_f64_n16384_b512_TN", kind="tlr_tlr", dtype="f64", N=16384, b=512,
            opA="T", opB="N", alpha=1.0, beta=1.0, budget=None, decay=0.9),
    4: dict(name="tlr_tlr_f32_n30000_b1024_ws1GiB", kind="tlr_tlr", dtype="f32", N=30000,
            b=1024, opA="N", opB="N", alpha=1.0, beta=0.0, budget=1 << 30, decay=1.0),
    5: dict(name="tlr_tlr_f64_n32768_b1024_heavy", kind="tlr_tlr", dtype="f64", N=32768,
            b=1024, opA="N", opB="N", alpha=1.0, beta=0.0, budget=None, decay=1.0),
}


def _offdiag_uniform(rng, q, lo, hi):
    R = np.zeros((q, q), dtype=np.int32)
    for i in range(q):
        for j in range(q):
            if i != j:
                R[i, j] = rng.integers(lo, hi + 1)
    return R


def config_ranks(c: int, stream: int) -> np.ndarray:
    """Rank table of operand A (stream 0) or B (stream 1) of workload c."""
    cfg = CONFIGS[c]
    q = len(tile_sizes(cfg["N"], cfg["b"]))
    rng = np.random.default_rng(1000 * c + stream)
    if c in (1,):
        return _offdiag_uniform(rng, q, 1, 16)
    if c == 2:
        return ranks_from_fn(q, q, lambda i, j: max(1, round(32 * math.exp(-abs(i - j) / 3))))
    if c == 3:
        R = np.zeros((q, q), dtype=np.int32)
        for i in range(q):
            for j in range(q):
                if i != j:
                    base = min(64, max(4, round(64 / (1 + abs(i - j)))))
                    R[i, j] = base + rng.integers(0, 5)
        return R
    if c == 4:
        return _offdiag_uniform(rng, q, 16, 128)
    if c == 5:
        n_off = q * (q - 1)
        heavy = set(int(x) for x in rng.choice(n_off, size=round(0.1 * n_off), replace=False))
        R = np.zeros((q, q), dtype=np.int32)
        t = 0
        for i in range(q):
            for j in range(q):
                if i == j:
                    continue
                R[i, j] = 256 if t in heavy else rng.integers(8, 33)
                t += 1
        return R
    raise KeyError(c)


def config_inputs(c: int, with_c: bool = True, dtype: Optional[str] = None):
    """(A, B, C_in) of workload c.  B is a TLRTiles or, for the TLR x dense
    workload, a dense (N, N) array; C_in is None when beta == 0 (or when
    ``with_c`` is False).  Dense arrays are indexed [row, col].  ``dtype``
    replaces the workload's element type (same draws, rounded to that type)."""
    cfg = CONFIGS[c]
    N, b = cfg["N"], cfg["b"]
    dt = dtype or cfg["dtype"]
    RA = config_ranks(c, 0)
    A = fill_values(np.random.default_rng(1000 * c + 2), N, N, b, RA, True, dt, cfg["decay"])
    if cfg["kind"] == "tlr_dense":
        B = on_grid(np.random.default_rng(1000 * c + 3).standard_normal((N, N)), dt)
    else:
        RB = config_ranks(c, 1)
        B = fill_values(np.random.default_rng(1000 * c + 3), N, N, b, RB, True, dt, cfg["decay"])
    C = None
    if with_c and cfg["beta"] != 0.0:
        C = on_grid(np.random.default_rng(1000 * c + 4).standard_normal((N, N)), dt)
    return A, B, C

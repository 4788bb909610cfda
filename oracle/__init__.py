"""CPU oracle for the Tile-Low-Rank GEMM  C <- alpha op(A) op(B) + beta C.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke entry point
and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
path; its only input dependency is the seeded generator package
``tlr_inputs`` (random numbers and per-tile arrangement, no arithmetic of the
method).

Contents
  reference   dense fp64 reconstruction of every tile and one BLAS matmul:
              the plain definition of the product.
  brute       the per-contraction-tile loop (coupling, right product, update)
              in pure-Python scalar loops, for tiny grids; it also counts the
              multiply-adds it performs for a chosen association order.
  plan_arith  rank-metadata arithmetic: panel rank sums, stage GEMM shapes,
              final-stage costs of both association orders, workspace sizes,
              useful-FLOP totals.
  unpack      reads the library's packed factor buffers back into tiles from
              the packing rules, independently of the package's packer.
  checks      invariant checks on a rectangle schedule (cover, disjointness,
              budget).
  recompress  the TLR-output product: the exact product, then every
              off-diagonal tile truncated by SVD to the smallest rank that
              meets a relative Frobenius tolerance; also dense-to-TLR
              compression.

Every function is pinned by the CPU tests (tests/test_oracle_*.py) to values
printed on the pages, closed forms, special cases and brute force.
"""
from . import reference, brute, plan_arith, unpack, checks, recompress  # noqa: F401

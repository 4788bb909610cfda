"""The seeded generator reproduces the rank tables of the five workloads.

Pinned values: rank sums of the seeded rank tables (computed once from the
generator specification and recorded with it), the rank formulas' ranges, and
the tile grids (q = ceil(N / b), last tile N - (q-1) b)."""
import numpy as np
import pytest

from tlr_inputs import CONFIGS, config_ranks, tile_sizes

PINS = {
    1: dict(sumA=497, sumB=443, q=8),
    2: dict(sumA=2010, q=16, rho=(82, 146)),
    3: dict(sumA=11200, sumB=11121, q=32, max=36),
    4: dict(sumA=61277, sumB=61468, q=30, last=304),
    5: dict(sumA=43456, sumB=43029, q=32, max=256, rho=(632, 2058)),
}


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_rank_pins(c):
    cfg, pin = CONFIGS[c], PINS[c]
    sizes = tile_sizes(cfg["N"], cfg["b"])
    assert len(sizes) == pin["q"]
    if "last" in pin:
        assert sizes[-1] == pin["last"]
    RA = config_ranks(c, 0)
    assert int(RA.sum()) == pin["sumA"]
    assert np.all(np.diag(RA) == 0)
    if "sumB" in pin:
        RB = config_ranks(c, 1)
        assert int(RB.sum()) == pin["sumB"]
        assert np.all(np.diag(RB) == 0)
    if "max" in pin:
        assert int(RA.max()) == pin["max"]
    if "rho" in pin:
        rho = RA.sum(axis=1)
        assert (int(rho.min()), int(rho.max())) == pin["rho"]


def test_heavy_tail_count():
    # 10 % of the 992 off-diagonal tiles at rank 256, the rest in [8, 32]
    for s in (0, 1):
        R = config_ranks(5, s)
        off = R[~np.eye(32, dtype=bool)]
        assert int((off == 256).sum()) == round(0.1 * 992)
        rest = off[off != 256]
        assert rest.min() >= 8 and rest.max() <= 32


def test_tile_sizes():
    assert tile_sizes(512, 64) == [64] * 8
    assert tile_sizes(30000, 1024) == [1024] * 29 + [304]
    assert tile_sizes(7, 3) == [3, 3, 1]
    assert tile_sizes(0, 3) == []

"""The schedule checker of the oracle accepts exact covers and rejects the rest.

"Tile-Low-Rank GEMM: Designing Storage Around the Contraction", section
"Association order and workspace": rectangles of output tiles write disjoint
parts of C and together cover it.  checks.covers_exactly_once must therefore
say True for a partition of the tile grid and False for an overlap, a gap,
an empty rectangle or one reaching outside the grid.  Each case below is
written out by hand."""
import pytest

from oracle import checks


@pytest.mark.parametrize("rects", [
    [(0, 3, 0, 4)],                                          # one rectangle, the whole grid
    [(0, 1, 0, 4), (1, 3, 0, 4)],                            # two row runs
    [(0, 3, 0, 2), (0, 2, 2, 4), (2, 3, 2, 4)],              # column block, then row runs
    [(2, 3, 2, 4), (0, 3, 0, 2), (0, 2, 2, 4)],              # same cover, any order
    [(i, i + 1, j, j + 1) for i in range(3) for j in range(4)],   # tile by tile
])
def test_exact_covers_accepted(rects):
    assert checks.covers_exactly_once(rects, 3, 4)


@pytest.mark.parametrize("rects,why", [
    ([(0, 2, 0, 4), (1, 3, 0, 4)], "tile row 1 covered twice"),
    ([(0, 3, 0, 2), (0, 3, 1, 4)], "tile column 1 covered twice"),
    ([(0, 3, 0, 4), (2, 3, 3, 4)], "one tile covered twice"),
    ([(0, 1, 0, 4), (2, 3, 0, 4)], "tile row 1 missing"),
    ([(0, 3, 0, 3)], "tile column 3 missing"),
    ([(0, 3, 0, 2), (0, 2, 2, 4)], "tile (2, 2) and (2, 3) missing"),
    ([], "nothing covered"),
    ([(0, 4, 0, 4)], "row range past the grid"),
    ([(0, 3, 0, 5)], "column range past the grid"),
    ([(-1, 3, 0, 4)], "negative row start"),
    ([(0, 3, 0, 4), (1, 1, 0, 4)], "empty row range"),
    ([(0, 3, 0, 4), (0, 3, 2, 2)], "empty column range"),
    ([(0, 3, 4, 0)], "reversed column range"),
])
def test_bad_covers_rejected(rects, why):
    assert not checks.covers_exactly_once(rects, 3, 4), why

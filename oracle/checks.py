"""Invariant checks of a schedule of output rectangles.

"Tile-Low-Rank GEMM: Designing Storage Around the Contraction", section
"Association order and workspace": under a workspace budget the scheduler
splits C into rectangles of output tiles; each rectangle holds the whole
reduction over k, so every tile of C is written by exactly one rectangle, and
each rectangle's intermediates must fit the budget.  The exact partition is a
heuristic the pages state only in prose, so these checks pin what must hold
for any valid schedule, not one particular partition.
"""
from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np


def covers_exactly_once(rects: Iterable[Tuple[int, int, int, int]], qm: int, qn: int) -> bool:
    """rects = (i0, i1, j0, j1) half-open tile ranges; True iff every output
    tile of the qm x qn grid lies in exactly one of them."""
    hits = np.zeros((qm, qn), dtype=np.int64)
    for (i0, i1, j0, j1) in rects:
        if not (0 <= i0 < i1 <= qm and 0 <= j0 < j1 <= qn):
            return False
        hits[i0:i1, j0:j1] += 1
    return bool(np.all(hits == 1))

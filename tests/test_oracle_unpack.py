"""The oracle's unpacker, pinned to buffers written by hand.

tests/golden/packed_tiny.json holds a 5 x 5 operand (b = 3, so a 3-wide and a
2-wide tile, dense diagonal, one rank-1 and one rank-2 tile) as flat packed
buffers typed in by hand from the packing rule of "Tile-Low-Rank GEMM:
Designing Storage Around the Contraction", section "Packing for the
contraction", with the tiles they must give back.  The worked example of the
same page fixes the panel widths: the inner panel of contraction tile 1 is
(16 + 48) x 256, so in a buffer whose every element holds its own column
index the tiles must start at the hand-listed columns below.  Neither test
uses the package's packer."""
import json
import os

import numpy as np

from oracle import unpack

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_packed_tiny_operand():
    g = json.load(open(os.path.join(GOLD, "packed_tiny.json")))
    t = unpack.unpack(g["rows"], g["cols"], g["b"], np.array(g["ranks"]), g["has_diag"],
                      np.array(g["outer"], float), np.array(g["inner"], float), np.array(g["diag"], float), "f64")
    e = g["expect"]
    assert np.array_equal(t.U[(0, 1)], e["U_0_1"]) and np.array_equal(t.U[(1, 0)], e["U_1_0"])
    assert np.array_equal(t.V[(1, 0)], e["V_1_0"]) and np.array_equal(t.V[(0, 1)], e["V_0_1"])
    assert np.array_equal(t.diag[0], e["D_0"]) and np.array_equal(t.diag[1], e["D_1"])
    assert set(t.U) == {(0, 1), (1, 0)} and set(t.V) == {(0, 1), (1, 0)}


def test_worked_example_panel_offsets():
    w = json.load(open(os.path.join(GOLD, "worked_example.json")))
    b = w["b"]
    R = np.array(w["A_ranks"])                     # 2 x 3 tiles, no dense diagonal
    ncols = int(R.sum())                           # 176 columns in each factor buffer
    assert ncols == sum(w["printed"]["rho"])
    # element (row, col) of each buffer holds col + row / 1000
    rows = np.arange(b)[:, None] / 1000.0
    flat = (np.arange(ncols)[None, :] + rows).T.ravel()          # column-major, leading dim b
    t = unpack.unpack(2 * b, 3 * b, b, R, False, flat, flat, None, "f64")
    # outer (U): tile row 0 holds 16 + 48 + 32 columns, then tile row 1 48 + 16 + 16
    u_start = {(0, 0): 0, (0, 1): 16, (0, 2): 64, (1, 0): 96, (1, 1): 144, (1, 2): 160}
    # inner (V): tile column 0 holds 16 + 48 (the printed (16+48) x 256 panel),
    # tile column 1 48 + 16, tile column 2 32 + 16
    v_start = {(0, 0): 0, (1, 0): 16, (0, 1): 64, (1, 1): 112, (0, 2): 128, (1, 2): 160}
    for key, c0 in u_start.items():
        r = int(R[key])
        assert np.array_equal(t.U[key], np.arange(c0, c0 + r)[None, :] + rows), key
    for key, c0 in v_start.items():
        r = int(R[key])
        assert np.array_equal(t.V[key], np.arange(c0, c0 + r)[None, :] + rows), key
    assert v_start[(1, 0)] + R[1, 0] == 16 + 48

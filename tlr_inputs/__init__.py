"""Seeded synthetic inputs for the Tile-Low-Rank GEMM.

This package only draws random numbers and arranges them per tile.  It holds
none of the product's arithmetic, so both the CPU oracle and the GPU path may
import it.
"""
from .gen import (TLRTiles, CONFIGS, TLR_OUT, basis_tlr, config_inputs, config_ranks, gaussian_sketch,
                  random_tlr, tile_sizes, tlr_out_inputs, ranks_from_fn, on_grid)

__all__ = ["TLRTiles", "CONFIGS", "TLR_OUT", "basis_tlr", "config_inputs", "config_ranks", "gaussian_sketch",
           "random_tlr", "tile_sizes", "tlr_out_inputs", "ranks_from_fn", "on_grid"]

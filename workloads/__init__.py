"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.  Holds input recipes and counting only; no attention arithmetic."""

from .bf16 import bf16_bits_to_f32, bf16_round, f32_to_bf16_bits
from .configs import CONFIGS, Config, Workload, make_workload, ones_bitmap, tile_grid
from . import accounting

__all__ = [
    "CONFIGS", "Config", "Workload", "make_workload", "ones_bitmap", "tile_grid",
    "accounting", "bf16_bits_to_f32", "bf16_round", "f32_to_bf16_bits",
]

"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no part of the attention method's arithmetic: only random draws, the
planted structure of the input recipe, per-head pattern maps and the named
workload shapes.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    STRUCTURED_LATENT,
    PlantInfo,
    planted_qkv,
    pattern_heads,
    grid_qkv,
    pattern_map,
    injected_vs_index,
    vertical_gain_for,
    config_kinds,
)

"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package holds only input generation: the five DiT-shaped configurations
(their sizes, block sizes, mask parameters and seeds) and the seeded random
draws.  It contains none of the attention method's arithmetic, so both the
CPU oracle and the GPU path can take their inputs from it without sharing
any computation.
"""
from .configs import CONFIGS, SWEEP_C3, MaskSpec, Config, MASK_DIAG, MASK_BAND, MASK_COGVIDEO3D, MASK_FULL, MASK_CUSTOM
from .gen import bf16_round, make_qkv, drift, sample_rows, make_cache, random_mask

__all__ = [
    "CONFIGS", "SWEEP_C3", "MaskSpec", "Config", "MASK_DIAG", "MASK_BAND", "MASK_COGVIDEO3D", "MASK_FULL", "MASK_CUSTOM",
    "bf16_round", "make_qkv", "drift", "sample_rows", "make_cache", "random_mask",
]

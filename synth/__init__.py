"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds only workload shapes and random-number generation.  It
contains none of the layer's arithmetic, so both the CPU oracle and the GPU
path may import it without sharing any of the method's code.
"""
from .configs import CONFIGS, LayerConfig, get_config
from .gen import (LayerWeights, bf16_round, bf16_bits, gen_rows, gen_weights,
                  gen_x_rows, gen_gamma)

__all__ = ["CONFIGS", "LayerConfig", "get_config", "LayerWeights", "bf16_round",
           "bf16_bits", "gen_rows", "gen_weights", "gen_x_rows", "gen_gamma"]

"""Seeded synthetic inputs for the SAF hybrid attention layer.

This package holds only random-number generation, rounding to the storage
dtype and the table of workload shapes. It contains none of the layer's
arithmetic, so both the float64 oracle (``oracle/``) and the HIP path's tests
and bench may draw from it without sharing any computation.
"""

from .configs import CONFIGS, Config, get_config
from .gen import Inputs, bf16_round, bf16_bits, bits_to_f32, make_inputs

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "Inputs",
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "make_inputs",
]

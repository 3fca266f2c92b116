"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package only draws random numbers and rounds them to bf16.  It holds none of the
method's arithmetic (no attention, scoring, allocation or quantisation), so that the CPU
oracle and the HIP path can both consume its arrays without sharing any code.
"""

from .configs import CONFIGS, WorkloadConfig, get_config
from .gen import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    make_config_inputs,
)

__all__ = [
    "CONFIGS",
    "WorkloadConfig",
    "get_config",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "make_inputs",
    "make_config_inputs",
]

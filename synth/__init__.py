"""Seeded synthetic input generators shared by the CPU oracle and the HIP path.

This package draws random numbers and formats them (fp32 -> bf16 rounding for
the bf16 workloads); it holds none of the draft-tree method's arithmetic.
"""
from .configs import CONFIGS, RoundConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_round, bf16_bits, make_inputs, RoundInputs,
)

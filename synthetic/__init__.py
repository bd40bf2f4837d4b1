"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package holds the workload shapes and the random-number draws only: it
contains none of the attention arithmetic.  Both sides of every parity check
take their inputs from here, so neither ever reads an input produced by the
other.
"""
from .configs import CONFIGS, MLAConfig, config
from .inputs import (Case, bf16_bits, bf16_to_f32, round_bf16, make_case,
                     make_weights, make_lengths, make_page_table, make_rows,
                     make_e4m3_rows, make_x, quiet_then_loud)

__all__ = [
    "CONFIGS", "MLAConfig", "config", "Case", "bf16_bits", "bf16_to_f32",
    "round_bf16", "make_case", "make_weights", "make_lengths",
    "make_page_table", "make_rows", "make_e4m3_rows", "make_x", "quiet_then_loud",
]

"""Seeded synthetic inputs for S2-Attn, shared by the tests, the bench and the oracle.

This package holds workload shapes and random draws only. It contains none of
the attention arithmetic: the GPU path and the CPU oracle each implement the
method on their own and meet only here, on identical input values.
"""

from .configs import BLOCK_CONFIGS, CONFIGS, BlockWorkload, Workload, workload
from .gen import bf16_bits, bf16_round, make_block_inputs, make_inputs

__all__ = ["BLOCK_CONFIGS", "CONFIGS", "BlockWorkload", "Workload", "workload", "bf16_round",
           "bf16_bits", "make_block_inputs", "make_inputs"]

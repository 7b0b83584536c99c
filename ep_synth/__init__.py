"""Seeded synthetic inputs for the MoE expert-parallel combine.

This package only draws random inputs (routing, routing weights, expert input
rows, expert weights, their fp8 encodings) and lays the dispatched rows out in
the grouped order the grouped GEMM consumes.  It holds none of the combine's
arithmetic and is shared by the oracle-side tests and the HIP-side tests/bench
as a source of identical bytes.
"""
from .configs import (CONFIGS, DEEPSEEK_DECODE, DEEPSEEK_PREFILL, QWEN3_MOE,
                      SKEWED_FP8, TINY, EpConfig, config_by_name)
from .generate import EpInputs, make_inputs, make_routing, make_up_inputs

__all__ = [
    "CONFIGS", "DEEPSEEK_DECODE", "DEEPSEEK_PREFILL", "QWEN3_MOE", "SKEWED_FP8",
    "TINY", "EpConfig", "config_by_name", "EpInputs", "make_inputs", "make_routing",
    "make_up_inputs",
]

"""Seeded synthetic inputs for the MoE expert-parallel combine.

This package only draws random inputs (routing, routing weights, expert input
rows keyed by pick, expert weights, their fp8 encodings).  It holds none of
the method's arithmetic (no locality test, no grouping): the oracle and the
HIP path each group the routing themselves and ask for the rows of their own
picks, so both see identical bytes for every pick.
"""
from .configs import (CONFIGS, DEEPSEEK_DECODE, DEEPSEEK_PREFILL, QWEN3_MOE,
                      SKEWED_FP8, TINY, EpConfig, config_by_name)
from .generate import (EpInputs, make_inputs, make_routing, make_tokens, make_up_weights,
                       make_weights, pick_rows, pick_up_rows)

__all__ = [
    "CONFIGS", "DEEPSEEK_DECODE", "DEEPSEEK_PREFILL", "QWEN3_MOE", "SKEWED_FP8",
    "TINY", "EpConfig", "config_by_name", "EpInputs", "make_inputs", "make_routing",
    "make_tokens", "make_up_weights", "make_weights", "pick_rows", "pick_up_rows",
]

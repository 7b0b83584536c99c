"""Named workload shapes for the MoE expert-parallel combine.

Each configuration fixes the geometry of one GPU's share of an expert-parallel
MoE down-projection + combine: R logical ranks, a slice of E_l local experts out
of E_g global ones, T tokens per source rank (equal to max_tokens_per_rank),
top_k picks per token, and the logical expert weight W_e of shape K x N whose
output rows are msg_bytes = 2N bytes (bf16).  The shapes follow DeepSeek-V3 and
Qwen3-MoE layer sizes; every value is synthetic.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class EpConfig:
    name: str
    n_ranks: int              # R: logical ranks (receive buffers), <= 8
    n_experts_global: int     # E_g
    n_experts_local: int      # E_l: experts owned by this GPU (n_experts_per_device)
    tokens_per_rank: int      # T = max_tokens_per_rank
    top_k: int
    k: int                    # GEMM reduction dim (expert intermediate width)
    n: int                    # GEMM output width (hidden size)
    dtype: str = "bf16"       # "bf16" or "fp8" (e4m3fn with 1x128 / 128x128 fp32 scales)
    routing: str = "uniform"  # "uniform" or "zipf"
    zipf_s: float = 1.2
    n_forced_empty: int = 0   # coldest local experts forced to receive no rows (zipf only)
    my_rank: int = 0
    seed: int = 0
    msg_bytes: int = 0        # 0 -> 2*n

    @property
    def msg(self) -> int:
        return self.msg_bytes if self.msg_bytes else 2 * self.n

    def replace(self, **kw) -> "EpConfig":
        return dataclasses.replace(self, **kw)


TINY = EpConfig("tiny", 2, 4, 2, 8, 2, 64, 128)
DEEPSEEK_DECODE = EpConfig("deepseek_decode", 8, 256, 32, 128, 8, 2048, 7168)
DEEPSEEK_PREFILL = EpConfig("deepseek_prefill", 8, 256, 32, 4096, 8, 2048, 7168)
QWEN3_MOE = EpConfig("qwen3_moe", 8, 128, 16, 1024, 8, 1536, 4096)
SKEWED_FP8 = EpConfig("skewed_fp8", 8, 256, 32, 2048, 8, 2048, 7168, dtype="fp8",
                      routing="zipf", zipf_s=1.2, n_forced_empty=4)

CONFIGS = {c.name: c for c in (TINY, DEEPSEEK_DECODE, DEEPSEEK_PREFILL, QWEN3_MOE, SKEWED_FP8)}


def config_by_name(name: str) -> EpConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}") from None

"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same entry points, same tiles), against the whole-step
oracle: the HIP path groups the routing itself (ep_group_local_picks), then
every receive-buffer byte, every count word, flag and counter, and every
combined output value is compared.  Integer results (grouping, placement,
counts, flags, counters, +0 of tokens without local picks) are exact; values
are within the stated tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

from gpu_helpers import compare_step, device_inputs, make_ctx, oracle_step  # noqa: E402

FULL = ["deepseek_decode", "deepseek_prefill", "qwen3_moe", "skewed_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_step(name):
    cfg = CONFIGS[name]
    print(f"[case] full size {name}", flush=True)
    inp = make_inputs(cfg)
    R, T, N = cfg.n_ranks, cfg.tokens_per_rank, cfg.n
    ctx = make_ctx(cfg)
    d = device_inputs(inp, ctx)
    out = torch.full((R, T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
             d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    del d
    print(f"[case] full size {name}: oracle", flush=True)
    ref = oracle_step(inp, epoch=ctx.epoch)
    off, src = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    assert np.array_equal(off, ref["offsets"]) and np.array_equal(src, ref["src_info"])
    print(f"[case] full size {name}: compare {int(off[-1])} rows, {R * T} tokens", flush=True)
    compare_step(ctx, ref, cfg, out, cfg.msg)

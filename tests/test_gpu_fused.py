"""The fused step (ep_grouped_gemm_scatter_combine): the GEMM with the sink
epilogue and the consumer combine in one launch, so the consumer workgroups
acquire rank completion (or each expert's count word) while other workgroups
of the same grid are still producing rows: the acquire-release election is
what orders them.  Checked against the oracle at every named parity shape and
at two full workloads, and over many consecutive steps whose receive buffers
are poisoned before each launch: a consumer that read a slot before its
producer's row was published would read the poison, and its output bits would
differ from the step's deterministic result."""
import numpy as np
import pytest
import torch

from ep_synth import CONFIGS, make_inputs
from gpu_helpers import (bits, compare_control, compare_step, device_inputs, make_ctx,
                         oracle_step)
from test_gpu_parity import CASES, _run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_step_matches_oracle(name):
    _run(CASES[name], fused=True)


@pytest.mark.parametrize("name", ["tiny", "multi_tile_256", "zipf_empty_experts",
                                  "decode_zipf_empty_experts", "fp8_multi_tile"])
def test_fused_per_expert_completion_matches_oracle(name):
    _run(CASES[name], epochs=2, fused=True, per_expert_release=True)


def test_fused_system_scope_matches_oracle():
    _run(CASES["multi_tile_256"], epochs=2, fused=True, system_scope=True)


@pytest.mark.parametrize("name", ["deepseek_decode", "qwen3_moe"])
def test_fused_full_size_step(name):
    cfg = CONFIGS[name]
    print(f"[case] fused full size {name}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    d = device_inputs(inp, ctx)
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
             d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"], fused=True)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    del d
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg)


LITMUS = {
    # rank-level election, agent scope: prefill-like ragged groups, several tiles
    "rank": (CASES["multi_tile_256"], {}),
    "rank_decode_tile": (CASES["decode_ragged"], {}),
    "rank_fp8": (CASES["fp8_wide_ragged"], {}),
    "per_expert": (CASES["zipf_empty_experts"], {"per_expert_release": True}),
    "system_scope": (CASES["many_experts_ragged"], {"system_scope": True}),
}


@pytest.mark.parametrize("name", sorted(LITMUS))
def test_fused_consumers_never_see_unpublished_rows(name, steps=2000):
    """Hundreds of fused steps in a row, each launched on receive buffers and
    outputs filled with poison (0xFF bytes: bf16 NaN) on the same stream: every
    step's output and control words must equal the first step's bit for bit
    (the first is checked against the oracle), the counters must re-arm, and no
    wait may time out."""
    cfg, kw = LITMUS[name]
    print(f"[case] litmus {name} {cfg} x{steps}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, flag_spin_limit=1 << 24, **kw)
    d = device_inputs(inp, ctx)
    R, T, N = cfg.n_ranks, cfg.tokens_per_rank, cfg.n
    out = torch.empty((R, T, N), dtype=torch.bfloat16, device="cuda")

    def step():
        for r in ctx.recv:
            r.fill_(0xFF)
        out.view(torch.int16).fill_(-1)
        ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
                 d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"], fused=True)

    step()
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref = oracle_step(inp, epoch=ctx.epoch, per_expert=kw.get("per_expert_release", False))
    compare_step(ctx, ref, cfg, out, cfg.msg)
    first = out.clone()
    El = cfg.n_experts_local
    counts = ctx.words[: El * R].clone()
    mismatch = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(1, steps):
        step()
        # device-side comparison, one host sync at the end
        mismatch += (out.view(torch.int16) != first.view(torch.int16)).sum()
        if kw.get("per_expert_release"):
            tag = (ctx.epoch & 0xFFFFFFFF) << 32
            mismatch += (ctx.words[: El * R] != (counts & 0xFFFFFFFF) + tag).sum()
        else:
            mismatch += (ctx.words[: El * R] != counts).sum()
            mismatch += (ctx.words[El * R:] != ctx.epoch).sum()
    torch.cuda.synchronize()
    assert ctx.query_error() == 0, "a consumer wait timed out"
    assert int(mismatch.item()) == 0, f"{int(mismatch.item())} values differ from the first step"
    assert torch.all(ctx.rank_counter == 0) and torch.all(ctx.tile_counter == 0)
    assert np.array_equal(bits(out), bits(first))

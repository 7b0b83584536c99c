"""The expert FFN end to end through the C ABI.  First form: the up-projection with SwiGLU
(ep_grouped_gemm_swiglu) writes H, which is the X of the down-projection with
the receive-buffer sink (ep_grouped_gemm_scatter), followed by the combine
(ep_combine_reduce).  The HIP side groups the routing itself and draws the X1
rows of its own picks; the oracle composes its own steps in the same way
(expert_swiglu, rounded to bf16, then the whole step on those rows).
Second form, from the tokens: ep_dispatch_rows gathers every local pick's
token row, then the same three calls.  Placement, counts and flags are
exact; values within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import CONFIGS, make_inputs
from gpu_helpers import compare_step, layout_picks, make_ctx, to_dev
from test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

CHAIN = {
    "multi_tile_256": CASES["multi_tile_256"],
    "zipf_empty_experts": CASES["zipf_empty_experts"],
    "many_experts_ragged": CASES["many_experts_ragged"],
    "qwen3_moe": CONFIGS["qwen3_moe"],
}


@pytest.mark.parametrize("name", sorted(CHAIN))
def test_up_projection_feeds_the_down_projection_and_its_sink(name):
    cfg = CHAIN[name]
    print(f"[case] chain {name} {cfg}", flush=True)
    inp = make_inputs(cfg)
    R, T, N, I = cfg.n_ranks, cfg.tokens_per_rank, cfg.n, cfg.k
    ctx = make_ctx(cfg)
    ids = to_dev(inp.topk_ids.astype(np.int32))
    tw = to_dev(inp.topk_w.astype(np.float32))
    offsets, src_info = ctx.group(ids)
    M = int(offsets[-1].item())
    x1 = to_dev(inp.up_rows(layout_picks(offsets, src_info, R, M)), torch.bfloat16)
    w1_h = inp.up_weights()
    w1 = to_dev(w1_h, torch.bfloat16)
    h = torch.empty((max(M, 1), I), dtype=torch.bfloat16, device="cuda")
    w = to_dev(inp.w, torch.bfloat16)
    out = torch.full((R, T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx.up_swiglu(x1 if M else None, w1, offsets, M, h if M else None)
    ctx.step(h if M else None, w, offsets, src_info, M, ids, tw, out)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0

    # the oracle's composition: its own grouping, its own X1 rows, H rounded to
    # bf16 once, then the whole step with H as the expert input rows
    off_o, src_o = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    x1_o = inp.up_rows(O.row_picks(off_o, src_o, R))
    h_o = O.f64_to_bf16(O.expert_swiglu(x1_o, w1_h, off_o, R).astype(np.float64))
    ref = O.run_step(topk_ids=inp.topk_ids, topk_w=inp.topk_w, x=h_o, w=inp.w, n_ranks=R,
                     n_experts_per_device=cfg.n_experts_local, top_k=cfg.top_k,
                     msg_bytes=cfg.msg, max_tokens_per_rank=T, my_rank=cfg.my_rank,
                     epoch=ctx.epoch)
    compare_step(ctx, ref, cfg, out, cfg.msg)


@pytest.mark.parametrize("name", ["multi_tile_256", "zipf_empty_experts", "qwen3_moe"])
def test_tokens_through_dispatch_up_projection_sink_and_combine(name):
    cfg = CHAIN[name]
    print(f"[case] token chain {name} {cfg}", flush=True)
    inp = make_inputs(cfg)
    R, T, N, I = cfg.n_ranks, cfg.tokens_per_rank, cfg.n, cfg.k
    ctx = make_ctx(cfg)
    ids = to_dev(inp.topk_ids.astype(np.int32))
    tw = to_dev(inp.topk_w.astype(np.float32))
    toks_h = inp.tokens()
    offsets, src_info = ctx.group(ids)
    M = int(offsets[-1].item())
    x1 = torch.empty((max(M, 1), N), dtype=torch.bfloat16, device="cuda")
    ctx.dispatch(to_dev(toks_h, torch.bfloat16), offsets, src_info, M, x1)
    w1_h = inp.up_weights()
    h = torch.empty((max(M, 1), I), dtype=torch.bfloat16, device="cuda")
    out = torch.full((R, T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx.up_swiglu(x1 if M else None, to_dev(w1_h, torch.bfloat16), offsets, M, h if M else None)
    ctx.step(h if M else None, to_dev(inp.w, torch.bfloat16), offsets, src_info, M, ids, tw, out)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0

    off_o, src_o = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    x1_o = O.dispatch_rows(toks_h, off_o, src_o, R)
    h_o = O.f64_to_bf16(O.expert_swiglu(x1_o, w1_h, off_o, R).astype(np.float64))
    ref = O.run_step(topk_ids=inp.topk_ids, topk_w=inp.topk_w, x=h_o, w=inp.w, n_ranks=R,
                     n_experts_per_device=cfg.n_experts_local, top_k=cfg.top_k,
                     msg_bytes=cfg.msg, max_tokens_per_rank=T, my_rank=cfg.my_rank,
                     epoch=ctx.epoch)
    compare_step(ctx, ref, cfg, out, cfg.msg)

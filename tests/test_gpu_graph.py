"""A step captured in a HIP graph (torch.cuda.CUDAGraph around the library's
calls on the capturing stream) and replayed.  With the epoch kept in device
memory (EP_FLAG_DEVICE_EPOCH) every replay is a fresh step: ep_advance_epoch,
the grouped GEMM with its sink and the combine (or the fused launch).  Each
replay, with the receive buffers and the output poisoned by eager work in
between, must reproduce the eager step bit for bit: the same slots and
combined output, flags (or tagged count words) carrying the replay's epoch,
re-armed counters and no error.  The eager step is itself checked against the
oracle.  A handle with the flag rejects a host epoch."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import make_inputs
from grouped_gemm_scatter_amd import EP_ERR_INVALID_ARG, EpError
from gpu_helpers import SENTINEL, compare_step, device_inputs, make_ctx, oracle_step
from test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

GRAPH_CASES = {
    "two_launch": ("multi_tile_256", {}),
    "two_launch_decode_tile": ("decode_ragged", {}),
    "two_launch_fp8": ("fp8_multi_tile", {}),
    "fused": ("multi_tile_256", {"fused": True}),
    "per_expert": ("zipf_empty_experts", {"per_expert": True}),
    "per_expert_fused": ("many_experts_ragged", {"per_expert": True, "fused": True}),
    "send_waves": ("tile_128_ragged", {"send_waves": 4}),
}


@pytest.mark.parametrize("name", sorted(GRAPH_CASES))
def test_replayed_step_equals_the_eager_step(name):
    case, kw = GRAPH_CASES[name]
    cfg = CASES[case]
    fused, per_expert = kw.get("fused", False), kw.get("per_expert", False)
    print(f"[case] graph {name} {cfg}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, device_epoch=True, per_expert_release=per_expert,
                   send_waves=kw.get("send_waves", 0))
    d = device_inputs(inp, ctx)
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")

    def step():
        ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
                 d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"], fused=fused)

    step()                                   # eager: epoch 1
    torch.cuda.synchronize()
    assert ctx.query_error() == 0 and int(ctx.epoch_word.item()) == 1
    compare_step(ctx, oracle_step(inp, epoch=1, per_expert=per_expert), cfg, out, cfg.msg, 1)
    ref_out = out.clone()
    ref_recv = [r.clone() for r in ctx.recv]
    counts = O.recv_counts(O.group_local_picks(inp.topk_ids, cfg.n_experts_local,
                                               cfg.my_rank)[0], cfg.n_ranks, cfg.n_experts_local)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    assert int(ctx.epoch_word.item()) == 1   # capturing runs nothing

    for r in range(4):
        out.fill_(float("nan"))
        for rb in ctx.recv:
            rb.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        epoch = 2 + r
        assert ctx.query_error() == 0, f"replay {r}"
        assert int(ctx.epoch_word.item()) == epoch
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {r}"
        for a, b in zip(ctx.recv, ref_recv):
            assert torch.equal(a, b), f"replay {r}: receive buffer"
        words = ctx.words.cpu().numpy().view(np.uint64)
        El, R = cfg.n_experts_local, cfg.n_ranks
        if per_expert:
            want = (np.uint64(epoch) << np.uint64(32)) | counts.astype(np.uint64)
            assert np.array_equal(words[:El * R], want.reshape(-1))
        else:
            assert np.array_equal(words[:El * R], counts.astype(np.uint64).reshape(-1))
            assert np.all(words[El * R:] == epoch)
            assert not ctx.rank_counter.any().item()
        assert not ctx.tile_counter.any().item()


def test_device_epoch_handle_rejects_a_host_epoch():
    cfg = CASES["tiny"]
    ctx = make_ctx(cfg, device_epoch=True)
    inp = make_inputs(cfg)
    d = device_inputs(inp, ctx)
    from grouped_gemm_scatter_amd import binding as B
    with pytest.raises(EpError) as e:
        B.ep_grouped_gemm_scatter(ctx.handle, d["x"], d["w"], None, None, d["offsets"],
                                  d["src_info"], d["m_total"], 0, None, 1)
    assert e.value.code == EP_ERR_INVALID_ARG
    with pytest.raises(EpError) as e:
        B.ep_combine_reduce(ctx.handle, d["topk_ids"], d["topk_w"], cfg.tokens_per_rank,
                            torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n),
                                        dtype=torch.bfloat16, device="cuda"), 1)
    assert e.value.code == EP_ERR_INVALID_ARG
    # a handle without the flag has no device epoch to advance
    plain = make_ctx(cfg)
    with pytest.raises(EpError):
        B.ep_advance_epoch(plain.handle)

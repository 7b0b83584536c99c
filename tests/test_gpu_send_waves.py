"""The grouped GEMM with dedicated send waves ("EpiloguePeerSink", SendWarps,
service, drain, shutdown; ep_combine_params.send_waves = 4) and the same
kernel with the sink inside the MFMA waves (EP_FLAG_SEND_TILE), through the C
ABI.

Each step is checked against the oracle element by element (placement,
counts, flags and counters bit-exact, values within tolerance).  Every kernel
of the library accumulates an output element over K in the same order with
the same MFMA instruction, so the send-wave kernel's receive buffers must also
equal the default kernel's byte for byte, which is checked at small sizes and
at the full prefill size.  The modes that share the epilogue (per-expert
completion, system scope, sink disabled, slot bounds check, consecutive
epochs) run through the send waves too."""
import numpy as np
import pytest
import torch

from ep_synth import CONFIGS, make_inputs
from grouped_gemm_scatter_amd import EP_ERR_UNSUPPORTED, EpError

pytestmark = pytest.mark.gpu

from gpu_helpers import (SENTINEL, assert_close, compare_step, device_inputs,  # noqa: E402
                         make_ctx, oracle_step, tol_for)
from test_gpu_parity import CASES  # noqa: E402

BF16_CASES = ["tiny", "multi_tile_256", "tile_128_ragged", "zipf_empty_experts", "single_rank",
              "no_local_rows", "many_experts_ragged", "decode_ragged", "decode_two_slices",
              "combine_rows_4096", "split_tail_mixed", "max_experts_top_k"]
MODES = {"send_waves": dict(send_waves=4), "sink_in_mfma_waves": dict(send_tile=True)}


def _step(cfg, epochs=1, **ctx_kw):
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, **ctx_kw)
    d = device_inputs(inp, ctx)
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    for _ in range(epochs):
        ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
                 d["topk_w"], out)
    torch.cuda.synchronize()
    return inp, ctx, d, out


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("name", BF16_CASES)
def test_step_matches_oracle(name, mode):
    cfg = CASES[name]
    print(f"[case] {mode} {name} {cfg}", flush=True)
    kw = MODES[mode]
    inp, ctx, d, out = _step(cfg, **kw)
    assert ctx.query_error() == 0
    assert ctx.gemm_tile(d["m_total"]) == (4 if "send_waves" in kw else 5, 128, 128)
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)


@pytest.mark.parametrize("name", ["multi_tile_256", "tile_128_ragged", "zipf_empty_experts",
                                  "decode_ragged", "split_tail_mixed"])
def test_receive_buffers_equal_the_default_kernels(name):
    cfg = CASES[name]
    print(f"[case] send waves vs default {name}", flush=True)
    ref_ctx = _step(cfg)[1]
    for kw in MODES.values():
        ctx = _step(cfg, **kw)[1]
        assert ctx.query_error() == 0
        for a, b in zip(ctx.recv, ref_ctx.recv):
            assert torch.equal(a, b)
        assert torch.equal(ctx.words, ref_ctx.words)


def test_consecutive_steps_advance_the_epoch():
    cfg = CASES["zipf_empty_experts"]
    inp, ctx, _, out = _step(cfg, epochs=3, send_waves=4)
    assert ctx.query_error() == 0 and ctx.epoch == 3
    compare_step(ctx, oracle_step(inp, epoch=3), cfg, out, cfg.msg, 3)


@pytest.mark.parametrize("name", ["tiny", "zipf_empty_experts", "many_experts_ragged"])
def test_per_expert_completion(name):
    cfg = CASES[name]
    print(f"[case] send waves, per-expert completion {name}", flush=True)
    inp, ctx, _, out = _step(cfg, send_waves=4, per_expert_release=True)
    assert ctx.query_error() == 0
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch, per_expert=True), cfg, out, cfg.msg,
                 ctx.epoch)


def test_system_scope():
    cfg = CASES["multi_tile_256"]
    inp, ctx, _, out = _step(cfg, send_waves=4, system_scope=True)
    assert ctx.query_error() == 0
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)


def test_sink_disabled_stores_local_c_only():
    cfg = CASES["tile_128_ragged"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, send_waves=4)
    d = device_inputs(inp, ctx)
    c = torch.empty((d["m_total"], cfg.n), dtype=torch.bfloat16, device="cuda")
    ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"],
                     p3_control=-1, c_local=c, epoch=1)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref_y = oracle_step(inp)["y_bits"]
    assert_close(c.cpu().view(torch.int16).numpy().view(np.uint16), ref_y, tol_for(cfg),
                 "local C")
    for rk in range(cfg.n_ranks):
        assert torch.all(ctx.recv[rk] == SENTINEL)
    assert torch.all(ctx.words == 0) and torch.all(ctx.tile_counter == 0)


def test_out_of_range_slot_is_latched_and_skipped():
    cfg = CASES["multi_tile_256"]
    inp = make_inputs(cfg)
    ref_ctx = make_ctx(cfg)
    ctx = make_ctx(cfg, send_waves=4)
    d = device_inputs(inp, ctx)
    d["src_info"][5, 0] = cfg.tokens_per_rank       # row 5's token index is out of range
    for c in (ref_ctx, ctx):
        c.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], epoch=1)
        torch.cuda.synchronize()
        assert c.query_error() == 1  # EP_ERR_SLOT_OOB
    # every other row lands where the default kernel puts it
    for a, b in zip(ctx.recv, ref_ctx.recv):
        assert torch.equal(a, b)


def test_fused_launch_is_unsupported():
    cfg = CASES["tiny"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, send_waves=4)
    d = device_inputs(inp, ctx)
    out = torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), dtype=torch.bfloat16,
                      device="cuda")
    with pytest.raises(EpError) as e:
        ctx.gemm_scatter_combine(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"],
                                 d["topk_ids"], d["topk_w"], out, epoch=1)
    assert e.value.code == EP_ERR_UNSUPPORTED


def test_full_prefill_size_equals_the_default_kernel():
    """deepseek_prefill at full size: the send-wave step's receive buffers,
    count words and combined output equal the default kernel's byte for byte
    (whose full-size step is checked against the oracle elsewhere)."""
    cfg = CONFIGS["deepseek_prefill"]
    print("[case] send waves, full-size prefill", flush=True)
    inp = make_inputs(cfg)
    outs, recvs, words = [], [], []
    for kw in ({}, dict(send_waves=4)):
        ctx = make_ctx(cfg, **kw)
        d = device_inputs(inp, ctx)
        out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                         dtype=torch.bfloat16, device="cuda")
        ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
                 d["topk_w"], out)
        torch.cuda.synchronize()
        assert ctx.query_error() == 0
        outs.append(out)
        recvs.append(ctx.recv)
        words.append(ctx.words)
        del d
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    for a, b in zip(*recvs):
        assert torch.equal(a, b)
    assert torch.equal(words[0], words[1])


def test_allocation_free_entry_point_runs_the_send_waves():
    """ep_grouped_gemm_scatter_noalloc on a send-wave handle (library-held
    counters) against ep_grouped_gemm_scatter on another, two calls in a row."""
    cfg = CASES["zipf_empty_experts"]
    inp = make_inputs(cfg)
    ref = make_ctx(cfg, send_waves=4)
    na = make_ctx(cfg, send_waves=4)
    d = device_inputs(inp, ref)
    for _ in range(2):
        for ctx, noalloc in ((ref, False), (na, True)):
            ctx.next_epoch()
            ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"],
                             noalloc=noalloc)
            torch.cuda.synchronize()
            assert ctx.query_error() == 0
        for a, b in zip(na.recv, ref.recv):
            assert torch.equal(a, b)
        assert torch.equal(na.words, ref.words)
        assert torch.all(na.tile_counter == 0) and torch.all(ref.tile_counter == 0)


@pytest.mark.parametrize("name", ["multi_tile_256", "tile_128_ragged", "decode_two_slices"])
def test_send_waves_on_slice_major_weights(name):
    """The send-wave kernel reading W as [E_l][K/64][N][64] (ep_pack_weights):
    against the oracle, and byte-equal to the same kernel on row-major W."""
    cfg = CASES[name]
    print(f"[case] send waves, slice-major W {name}", flush=True)
    inp = make_inputs(cfg)
    row = _step(cfg, send_waves=4)[1]
    ctx = make_ctx(cfg, send_waves=4, w_slice_major=True)
    d = device_inputs(inp, ctx)
    w = ctx.pack_weights(d["w"])
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    ctx.step(d["x"], w, d["offsets"], d["src_info"], d["m_total"], d["topk_ids"], d["topk_w"],
             out)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)
    for a, b in zip(ctx.recv, row.recv):
        assert torch.equal(a, b)

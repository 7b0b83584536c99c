"""Tile trace (EP_FLAG_TRACE) through the C ABI: a traced step still matches
the oracle, its records tile every local row x output column exactly once
(balanced bf16 row tiles, decode and fp8 tiles), and a buffer shorter than the
launch's tile count is never written past its end."""
import numpy as np
import pytest
import torch

from ep_synth import make_inputs
from gpu_helpers import compare_step, device_inputs, make_ctx, oracle_step
from test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


def _step(ctx, cfg, inp, d):
    out = torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), dtype=torch.bfloat16,
                      device="cuda")
    ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
             d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    return out


# balanced bf16 row tiles; empty experts; decode tiles; fp8 tiles; fp8 row
# bands of a hot expert; row tiles of 256 and 288 rows in one launch
@pytest.mark.parametrize("name", ["multi_tile_256", "zipf_empty_experts", "decode_ragged",
                                  "fp8_wide_ragged", "fp8_hot_expert_bands",
                                  "split_tail_mixed"])
def test_trace_records_tile_the_output_once(name):
    cfg = CASES[name]
    print(f"[case] trace {name}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, trace_records=8192)
    d = device_inputs(inp, ctx)
    ctx.reset_trace()
    out = _step(ctx, cfg, inp, d)
    ref = oracle_step(inp, epoch=ctx.epoch)
    compare_step(ctx, ref, cfg, out, cfg.msg, ctx.epoch)

    tab = ctx.trace_table()
    R = cfg.n_ranks
    off = ref["offsets"]
    cover = np.zeros((d["m_total"], cfg.n), dtype=np.int8)
    for m0, n0, e, rows, cols in zip(tab["m0"], tab["n0"], tab["expert"], tab["rows"],
                                     tab["cols"]):
        g0, g1 = int(off[e * R]), int(off[(e + 1) * R])
        assert rows > 0 and g0 <= m0 and m0 + rows <= g1, (m0, rows, e, g0, g1)
        assert cols in (128, 256) and n0 % cols == 0 and n0 + cols <= cfg.n
        cover[m0:m0 + rows, n0:n0 + cols] += 1
    assert np.all(cover == 1), "trace records do not tile the output exactly once"
    if name == "split_tail_mixed":
        # rows spread evenly: tiles of eight and of nine 32-row blocks
        assert tab["rows"].max() > 256 and tab["rows"].min() > 200
    assert np.all(tab["t_end"] >= tab["t_start"]) and np.all(tab["t_start"] > 0)


def test_trace_past_the_buffer_is_dropped():
    from grouped_gemm_scatter_amd import binding as B
    cfg = CASES["multi_tile_256"]
    print("[case] trace capacity 3", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, trace_records=3 + 16)
    d = device_inputs(inp, ctx)
    # the library sees the first 3 records; the other 16 are a guard
    B.ep_combine_destroy(ctx.handle)
    ctx.handle = B.ep_combine_init(ctx.params, ctx.recv, ctx.words, ctx.rank_counter,
                                   ctx.tile_counter, ctx.error_word, ctx.trace[:3])
    ctx.trace.zero_()
    ctx.trace[3:] = -1
    _step(ctx, cfg, inp, d)
    t = ctx.trace.cpu().numpy()
    assert np.all(t[3:] == -1), "a record was written past trace_records"
    assert np.all(t[:3, 2] > 0), "slots 0..2 hold the first three tiles"

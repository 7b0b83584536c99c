"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, on seeded inputs small enough for the oracle (several tiles, ragged
group tails, empty experts, padding, several ranks)."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import TINY, make_inputs

pytestmark = pytest.mark.gpu

from gpu_helpers import (SENTINEL, assert_close, bits, compare_control, compare_step,  # noqa: E402
                         device_inputs, make_ctx, oracle_step, tol_for)


def _run(cfg, msg_bytes=None, epochs=1, fused=False, **ctx_kw):
    print(f"[case] {cfg}", flush=True)
    inp = make_inputs(cfg)
    msg = msg_bytes or cfg.msg
    ctx = make_ctx(cfg, msg_bytes=msg, **ctx_kw)
    d = device_inputs(inp, ctx)
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    for _ in range(epochs):
        ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
                 d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"], fused=fused)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref = oracle_step(inp, msg_bytes=msg, epoch=ctx.epoch,
                      per_expert=ctx_kw.get("per_expert_release", False))
    compare_step(ctx, ref, cfg, out, msg, ctx.epoch)
    return ctx, inp, ref, out


CASES = {
    "tiny": TINY,
    "multi_tile_256": TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4,
                                   tokens_per_rank=384, top_k=4, k=512, n=512, my_rank=1, seed=11),
    "tile_128_ragged": TINY.replace(n_ranks=3, n_experts_global=9, n_experts_local=3,
                                    tokens_per_rank=200, top_k=3, k=192, n=384, my_rank=2, seed=12),
    "zipf_empty_experts": TINY.replace(n_ranks=8, n_experts_global=64, n_experts_local=8,
                                       tokens_per_rank=256, top_k=6, k=256, n=256,
                                       routing="zipf", n_forced_empty=2, seed=13),
    "single_rank": TINY.replace(n_ranks=1, n_experts_global=3, n_experts_local=3,
                                tokens_per_rank=300, top_k=2, k=128, n=256, seed=14),
    "no_local_rows": TINY.replace(n_ranks=2, n_experts_global=8, n_experts_local=4,
                                  tokens_per_rank=16, top_k=2, k=64, n=128, routing="zipf",
                                  n_forced_empty=4, seed=15),
    "many_experts_ragged": TINY.replace(n_ranks=8, n_experts_global=64, n_experts_local=8,
                                       tokens_per_rank=64, top_k=8, k=512, n=512, my_rank=5,
                                       seed=19),
    # at most 48 rows per local expert on average: the 64 x 128 decode tile
    # (three K slices in flight); K = 320, 64 and 128 give 5, 1 and 2 slices;
    # the zipf case holds experts of 0, 14-27, 60 and 79 rows (two row tiles)
    "decode_ragged": TINY.replace(n_ranks=8, n_experts_global=64, n_experts_local=8,
                                  tokens_per_rank=32, top_k=8, k=320, n=512, my_rank=2,
                                  seed=21),
    "decode_zipf_empty_experts": TINY.replace(n_ranks=4, n_experts_global=32, n_experts_local=8,
                                              tokens_per_rank=40, top_k=4, k=64, n=256,
                                              routing="zipf", n_forced_empty=3, seed=22),
    "decode_two_slices": TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4,
                                      tokens_per_rank=24, top_k=2, k=128, n=768, my_rank=3,
                                      seed=23),
    "fp8_multi_tile": TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4,
                                   tokens_per_rank=300, top_k=4, k=384, n=384, my_rank=3,
                                   dtype="fp8", seed=17),
    "fp8_zipf_empty_experts": TINY.replace(n_ranks=8, n_experts_global=64, n_experts_local=8,
                                           tokens_per_rank=256, top_k=6, k=256, n=256,
                                           routing="zipf", n_forced_empty=2, dtype="fp8", seed=18),
    # one hot expert of 10 row tiles (the fp8 item order walks it in bands of
    # four row tiles: two whole bands and a partial one), an empty expert
    "fp8_hot_expert_bands": TINY.replace(n_ranks=2, n_experts_global=8, n_experts_local=4,
                                         tokens_per_rank=1600, top_k=2, k=256, n=512,
                                         routing="zipf", n_forced_empty=1, dtype="fp8", seed=29),
    # N a multiple of 256: the 256 x 256 fp8 tile; three K slices (odd count)
    "fp8_wide_ragged": TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4,
                                    tokens_per_rank=300, top_k=4, k=384, n=512, my_rank=2,
                                    dtype="fp8", seed=24),
    # combine row widths: two waves share a token, with column ranges of 256,
    # 320 and 480 16-byte chunks (4 chunks per lane, 5 of an 8-chunk pass and
    # 7.5, ragged); the fused consumer takes whole rows (8, 10 of 14, and 15: a
    # second, ragged pass)
    "combine_rows_4096": TINY.replace(n_ranks=2, n_experts_global=4, n_experts_local=2,
                                      tokens_per_rank=48, top_k=2, k=64, n=4096, seed=25),
    "combine_rows_5120": TINY.replace(n_ranks=3, n_experts_global=6, n_experts_local=2,
                                      tokens_per_rank=40, top_k=3, k=64, n=5120, my_rank=1,
                                      seed=26),
    "combine_rows_7680": TINY.replace(n_ranks=2, n_experts_global=4, n_experts_local=2,
                                      tokens_per_rank=40, top_k=2, k=128, n=7680, my_rank=1,
                                      seed=27),
    # the largest local expert count (256: the work table, the finished-expert
    # set of eight words) and pick count (64: every lane of the combine's waves
    # holds a pick), a few rows per expert on the small-row-group tile
    "max_experts_top_k": TINY.replace(n_ranks=2, n_experts_global=512, n_experts_local=256,
                                      tokens_per_rank=48, top_k=64, k=128, n=256, my_rank=1,
                                      seed=31),
    # wide rows and a deep K: 64 K slices per tile, 32 KB rows: two waves of
    # 16 chunks per lane (two passes of the 14-chunk form, the second ragged)
    "wide_rows_deep_k": TINY.replace(n_ranks=2, n_experts_global=4, n_experts_local=2,
                                     tokens_per_rank=64, top_k=2, k=4096, n=16384, seed=32),
    # 2400 rows per local expert: 75 row blocks spread over nine row tiles
    # of eight or nine blocks (256 or 288 rows), 576 items on a 256-workgroup
    # grid (a partial third round)
    "split_tail_mixed": TINY.replace(n_ranks=4, n_experts_global=8, n_experts_local=4,
                                     tokens_per_rank=2400, top_k=2, k=64, n=4096, seed=28),
    # many tokens and 7680-wide rows: 7.5 chunks per lane in one ragged pass of
    # the 8-chunk form (two waves per token), 15 in the fused consumer
    "combine_rows_7680_many_tokens": TINY.replace(n_ranks=2, n_experts_global=4,
                                                  n_experts_local=2, tokens_per_rank=1024,
                                                  top_k=2, k=64, n=7680, my_rank=1, seed=33),
    # many tokens and 16384-wide rows: column ranges of 1024 chunks (16 per
    # lane: a second, ragged pass of the 14-chunk form), 32 per lane in the
    # fused consumer (three passes)
    "combine_rows_16384_many_tokens": TINY.replace(n_ranks=2, n_experts_global=4,
                                                   n_experts_local=2, tokens_per_rank=768,
                                                   top_k=2, k=64, n=16384, seed=34),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_matches_oracle(name):
    _run(CASES[name])


def test_padded_messages_leave_padding_untouched():
    cfg = CASES["tile_128_ragged"]
    _run(cfg, msg_bytes=cfg.msg + 64)


def test_consecutive_steps_advance_the_epoch():
    ctx, *_ = _run(CASES["multi_tile_256"], epochs=3)
    assert ctx.epoch == 3
    assert np.all(ctx.flags.cpu().numpy() == 3)


def test_system_scope_flag():
    _run(CASES["tiny"], system_scope=True)


def test_identity_weights_are_bit_exact():
    cfg = TINY.replace(n_ranks=2, n_experts_global=4, n_experts_local=2, tokens_per_rank=300,
                       top_k=2, k=256, n=256, seed=16)
    inp = make_inputs(cfg)
    eye = torch.eye(256, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    inp.w = np.ascontiguousarray(np.stack([eye, eye]))
    ctx = make_ctx(cfg)
    d = device_inputs(inp, ctx)
    out = torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), dtype=torch.bfloat16, device="cuda")
    ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
             d["topk_w"], out)
    torch.cuda.synchronize()
    ref = oracle_step(inp, epoch=1)
    for rk in range(cfg.n_ranks):
        assert np.array_equal(ctx.recv[rk].cpu().numpy(), ref["recv_bufs"][rk])


def test_sink_disabled_stores_local_c_only():
    cfg = CASES["multi_tile_256"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    d = device_inputs(inp, ctx)
    c = torch.empty((d["m_total"], cfg.n), dtype=torch.bfloat16, device="cuda")
    ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"],
                     p3_control=-1, c_local=c, epoch=1)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref_y = oracle_step(inp)["y_bits"]        # rows in the oracle's own grouped order
    assert_close(c.cpu().view(torch.int16).numpy().view(np.uint16), ref_y, tol_for(cfg), "local C")
    for rk in range(cfg.n_ranks):
        assert torch.all(ctx.recv[rk] == SENTINEL)
    assert torch.all(ctx.words == 0) and torch.all(ctx.tile_counter == 0)


def test_standalone_signals_follow_the_election_model():
    cfg = TINY.replace(n_ranks=4, n_experts_local=3, n_experts_global=12)
    ctx = make_ctx(cfg)
    R, El = 4, 3
    rng = np.random.default_rng(0)
    pairs = [(e, rk) for e in range(El) for rk in range(R)]
    order = rng.permutation(len(pairs))
    e = np.array([pairs[i][0] for i in order], np.int32)
    rk = np.array([pairs[i][1] for i in order], np.int32)
    val = rng.integers(0, 1 << 40, len(pairs)).astype(np.int64)
    model = O.ElectionModel(R, El, epoch=9)
    for i in range(len(pairs)):
        model.signal(int(e[i]), int(rk[i]), int(val[i]))
    ctx.signal(torch.from_numpy(e).cuda(), torch.from_numpy(rk).cuda(),
               torch.from_numpy(val).cuda(), epoch=9)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    assert np.array_equal(ctx.words.cpu().numpy().view(np.uint64), model.words)
    assert torch.all(ctx.rank_counter == 0)


@pytest.mark.parametrize("name", ["tiny", "multi_tile_256", "zipf_empty_experts",
                                  "decode_zipf_empty_experts", "fp8_multi_tile",
                                  "max_experts_top_k"])
def test_per_expert_completion_matches_oracle(name):
    # every count word is its own release store tagged with the step; the
    # combine acquires the E_l words of each rank (no election, no flags)
    _run(CASES[name], epochs=2, per_expert_release=True)


def test_per_expert_standalone_signals_tag_each_word():
    cfg = TINY.replace(n_ranks=4, n_experts_local=3, n_experts_global=12)
    ctx = make_ctx(cfg, per_expert_release=True)
    R, El = 4, 3
    rng = np.random.default_rng(1)
    pairs = [(e, rk) for e in range(El) for rk in range(R)]
    order = rng.permutation(len(pairs))
    e = np.array([pairs[i][0] for i in order], np.int32)
    rk = np.array([pairs[i][1] for i in order], np.int32)
    val = rng.integers(0, 1 << 31, len(pairs)).astype(np.int64)
    epoch = (1 << 33) + 5          # only the low 32 bits form the tag
    expect = np.zeros(El * R + R, dtype=np.uint64)
    for i in range(len(pairs)):
        expect[O.recv_count_index(int(e[i]), int(rk[i]), R)] = O.tagged_count(int(val[i]), epoch)
    ctx.signal(torch.from_numpy(e).cuda(), torch.from_numpy(rk).cuda(),
               torch.from_numpy(val).cuda(), epoch=epoch)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    assert np.array_equal(ctx.words.cpu().numpy().view(np.uint64), expect)
    assert torch.all(ctx.rank_counter == 0)


def test_per_expert_missing_word_times_out_for_its_rank_only():
    cfg = TINY.replace(n_ranks=2, n_experts_local=2, n_experts_global=4)
    ctx = make_ctx(cfg, flag_spin_limit=2000, per_expert_release=True)
    # rank 1 gets only one of its two count words
    e = torch.tensor([0, 1, 0], dtype=torch.int32, device="cuda")
    rk = torch.tensor([0, 0, 1], dtype=torch.int32, device="cuda")
    v = torch.zeros(3, dtype=torch.int64, device="cuda")
    ctx.signal(e, rk, v, epoch=1)
    ids = torch.full((2, cfg.tokens_per_rank, cfg.top_k), 3, dtype=torch.int32, device="cuda")
    tw = torch.zeros((2, cfg.tokens_per_rank, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.full((2, cfg.tokens_per_rank, cfg.n), 7.0, dtype=torch.bfloat16, device="cuda")
    ctx.combine(ids, tw, out, epoch=1)
    assert ctx.query_error() == 2  # EP_ERR_FLAG_TIMEOUT
    assert torch.all(out[1] == 7.0)
    assert torch.all(out[0] == 0.0)
    assert ctx.flags.cpu().tolist() == [0, 0]


def test_missing_signal_times_out_without_touching_output():
    cfg = TINY.replace(n_ranks=2, n_experts_local=2, n_experts_global=4)
    ctx = make_ctx(cfg, flag_spin_limit=2000)
    # rank 1 gets only one of its two expert signals: its flag never flips
    e = torch.tensor([0, 1, 0], dtype=torch.int32, device="cuda")
    rk = torch.tensor([0, 0, 1], dtype=torch.int32, device="cuda")
    v = torch.zeros(3, dtype=torch.int64, device="cuda")
    ctx.signal(e, rk, v, epoch=1)
    # every pick names global expert 3, which is not local: rank 0 combines to zeros
    ids = torch.full((2, cfg.tokens_per_rank, cfg.top_k), 3, dtype=torch.int32, device="cuda")
    tw = torch.zeros((2, cfg.tokens_per_rank, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.full((2, cfg.tokens_per_rank, cfg.n), 7.0, dtype=torch.bfloat16, device="cuda")
    ctx.combine(ids, tw, out, epoch=1)
    err = ctx.query_error()
    assert err == 2  # EP_ERR_FLAG_TIMEOUT
    assert torch.all(out[1] == 7.0)          # rank 1 untouched
    assert torch.all(out[0] == 0.0)          # rank 0 combined: no local pick gives +0
    assert ctx.flags.cpu().tolist() == [1, 0]


def test_out_of_range_slot_is_latched_and_skipped():
    cfg = CASES["tiny"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    d = device_inputs(inp, ctx)
    d["src_info"][0, 0] = cfg.tokens_per_rank       # row 0's token index is out of range
    M = d["m_total"]
    ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], M, epoch=1)
    assert ctx.query_error() == 1  # EP_ERR_SLOT_OOB
    ref = oracle_step(inp)
    # every other row still lands; the bad row's intended slot keeps the sentinel
    _, rk0 = O.row_owner(ref["offsets"], cfg.n_ranks, 0)
    ok_rows = 0
    for m in range(1, M):
        _, rk = O.row_owner(ref["offsets"], cfg.n_ranks, m)
        t, k = ref["src_info"][m]
        o = O.recv_slot_offset(int(t), int(k), 0, cfg.top_k, cfg.msg)
        got = ctx.recv[rk][o:o + 2 * cfg.n].cpu().numpy().view("<u2")
        assert_close(got, ref["recv_bufs"][rk][o:o + 2 * cfg.n].view("<u2"), 2e-2, f"row {m}")
        ok_rows += 1
    t, k = ref["src_info"][0]
    o = O.recv_slot_offset(int(t), int(k), 0, cfg.top_k, cfg.msg)
    assert torch.all(ctx.recv[rk0][o:o + 2 * cfg.n] == SENTINEL)
    assert ok_rows == M - 1


def test_inconsistent_offsets_do_nothing():
    cfg = CASES["tiny"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    d = device_inputs(inp, ctx)
    bad = d["offsets"].clone()
    bad[-1] += 1                                # no longer equals m_total
    ctx.gemm_scatter(d["x"], d["w"], bad, d["src_info"], d["m_total"], epoch=1)
    assert ctx.query_error() == 4  # EP_ERR_BAD_GROUP
    for rk in range(cfg.n_ranks):
        assert torch.all(ctx.recv[rk] == SENTINEL)
    assert torch.all(ctx.words == 0)


def _epilogue_pattern_bufs(inp, ref, msg):
    """Receive buffers after an epilogue-only launch: every local row m carries
    the exact bf16 values (m*131 + n*7) mod 256 at the oracle's slot; all other
    bytes keep the sentinel."""
    cfg = inp.cfg
    cap = cfg.tokens_per_rank * cfg.top_k * msg
    bufs = [np.full(cap, SENTINEL, dtype=np.uint8) for _ in range(cfg.n_ranks)]
    off, src = ref["offsets"], ref["src_info"]
    n = np.arange(cfg.n, dtype=np.int64)
    for m in range(int(off[-1])):
        _, rk = O.row_owner(off, cfg.n_ranks, m)
        o = O.recv_slot_offset(int(src[m][0]), int(src[m][1]), 0, cfg.top_k, msg)
        vals = ((m * 131 + n * 7) & 255).astype(np.float32)      # exact in bf16
        bits = (vals.view(np.uint32) >> 16).astype("<u2")
        bufs[rk][o:o + 2 * cfg.n] = bits.view(np.uint8)
    return bufs


@pytest.mark.parametrize("name", ["multi_tile_256", "tile_128_ragged", "zipf_empty_experts",
                                  "decode_ragged", "fp8_multi_tile", "fp8_wide_ragged"])
def test_epilogue_only_mode_places_the_pattern_and_signals(name):
    """EP_FLAG_EPILOGUE_ONLY (the scatter-timing mode): same placement, counts,
    flags and counter re-arm as a full step, with known exact row values."""
    cfg = CASES[name]
    print(f"[case] epilogue-only {cfg}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, epilogue_only=True)
    d = device_inputs(inp, ctx)
    for _ in range(2):
        ctx.next_epoch()
        ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"],
                         x_scale=d["x_scale"], w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref = oracle_step(inp, epoch=ctx.epoch)
    want = _epilogue_pattern_bufs(inp, ref, cfg.msg)
    for rk in range(cfg.n_ranks):
        got = ctx.recv[rk].cpu().numpy()
        assert np.array_equal(got, want[rk]), f"rank {rk}: receive buffer differs"
    words = ctx.words.cpu().numpy().view(np.uint64)
    assert np.array_equal(words, ref["control"]["words"]), "count words / flags differ"
    assert np.all(ctx.rank_counter.cpu().numpy() == 0)
    assert np.all(ctx.tile_counter.cpu().numpy() == 0)


@pytest.mark.parametrize("name", ["multi_tile_256", "decode_ragged", "fp8_multi_tile"])
def test_fewer_tokens_than_capacity(name):
    """tokens_per_rank below max_tokens_per_rank: the routing covers the first
    T tokens of each rank, slots of tokens past T keep the sentinel, and the
    combine reads and writes exactly T tokens per rank."""
    base = CASES[name]
    T_max = base.tokens_per_rank
    cfg = base.replace(tokens_per_rank=(2 * T_max) // 3 + 1)
    print(f"[case] fewer tokens {cfg} capacity {T_max}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, max_tokens=T_max)
    d = device_inputs(inp, ctx)
    # the output holds R*T rows, followed here by guard rows the combine must not touch
    R, T, N = cfg.n_ranks, cfg.tokens_per_rank, cfg.n
    whole = torch.full((R * T_max * N,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = whole[: R * T * N].view(R, T, N)
    out.fill_(float("nan"))
    guard = whole[R * T * N:]
    ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
             d["topk_w"], out, x_scale=d["x_scale"], w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref = oracle_step(inp, epoch=ctx.epoch, max_tokens=T_max)
    compare_step(ctx, ref, cfg, out, cfg.msg, max_tokens=T_max)
    assert torch.all(guard == 3.0)


@pytest.mark.parametrize("name", ["tiny", "combine_rows_5120", "combine_rows_7680",
                                  "zipf_empty_experts", "fp8_wide_ragged"])
def test_combine_is_bit_exact_on_the_oracles_slots(name):
    """The consumer combine alone, on receive buffers holding the oracle's own
    slot rows and flags published by standalone signals carrying the oracle's
    counts: both sides sum w * slot with one binary32 fused multiply-add per
    local pick in ascending pick order, so every output bit must agree."""
    cfg = CASES[name]
    print(f"[case] combine on oracle slots {cfg}", flush=True)
    inp = make_inputs(cfg)
    ref = oracle_step(inp, epoch=1)
    ctx = make_ctx(cfg)
    for rk in range(cfg.n_ranks):
        ctx.recv[rk].copy_(torch.from_numpy(ref["recv_bufs"][rk]))
    R, El = cfg.n_ranks, cfg.n_experts_local
    e = torch.arange(El, dtype=torch.int32).repeat_interleave(R).cuda()
    rk = torch.arange(R, dtype=torch.int32).repeat(El).cuda()
    counts = torch.from_numpy(ref["control"]["words"][:El * R].astype(np.int64)).cuda()
    ctx.signal(e, rk, counts, epoch=1)
    out = torch.full((R, cfg.tokens_per_rank, cfg.n), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    ids = torch.from_numpy(inp.topk_ids.astype(np.int32)).cuda()
    tw = torch.from_numpy(inp.topk_w).cuda()
    ctx.combine(ids, tw, out, epoch=1)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    got = bits(out)
    diff = np.argwhere(got != ref["out_bits"])
    assert diff.size == 0, f"{len(diff)} output values differ; first at {diff[:5].tolist()}"
    compare_control(ctx, ref)


def test_per_expert_mode_rejects_epochs_without_a_tag():
    """With per-expert completion the count words carry the epoch's low 32
    bits: an epoch whose low half is zero would match zeroed words, so every
    step call rejects it on the host before any launch."""
    from grouped_gemm_scatter_amd import EP_ERR_INVALID_ARG, EpError
    cfg = CASES["tiny"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg, per_expert_release=True)
    d = device_inputs(inp, ctx)
    out = torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), dtype=torch.bfloat16,
                      device="cuda")
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    for call in (lambda: ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"],
                                          d["m_total"], epoch=1 << 32),
                 lambda: ctx.signal(one, one, one.to(torch.int64), epoch=5 << 32),
                 lambda: ctx.combine(d["topk_ids"], d["topk_w"], out, epoch=1 << 32)):
        with pytest.raises(EpError) as ei:
            call()
        assert ei.value.code == EP_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    assert torch.all(ctx.words == 0)

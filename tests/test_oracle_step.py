"""Pins of the oracle's scatter, counts, completion contract and combine."""
import itertools
from collections import Counter

import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import TINY, make_inputs, make_routing


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _geom(cfg, msg=None):
    return dict(n_ranks=cfg.n_ranks, n_experts_per_device=cfg.n_experts_local,
                top_k=cfg.top_k, msg_bytes=msg or cfg.msg,
                max_tokens_per_rank=cfg.tokens_per_rank, my_rank=cfg.my_rank)


@pytest.mark.parametrize("variant", [
    dict(),
    dict(n_ranks=4, n_experts_global=12, n_experts_local=3, tokens_per_rank=16, top_k=3, my_rank=2, seed=5),
    dict(n_ranks=3, n_experts_global=6, n_experts_local=2, tokens_per_rank=9, top_k=4, my_rank=1, seed=9),
])
@pytest.mark.parametrize("pad", [0, 32])
def test_identity_step_places_every_row_exactly_once(variant, pad):
    """W = I and X rows that spell their own (rk, t, k): each local slot must
    hold exactly its pick's row, every other byte keeps the sentinel."""
    cfg = TINY.replace(k=128, n=128, **variant)
    ids, tw = make_routing(cfg)
    offsets, src = O.group_local_picks(ids, cfg.n_experts_local, cfg.my_rank)
    M = int(offsets[-1])
    x = np.zeros((M, cfg.k), np.float32)
    for m in range(M):
        e, rk = O.row_owner(offsets, cfg.n_ranks, m)
        x[m, :4] = [rk + 1, src[m][0] + 1, src[m][1] + 1, e + 1]
    w = np.stack([np.eye(cfg.n, cfg.k)] * cfg.n_experts_local)
    g = _geom(cfg, cfg.msg + pad)
    res = O.run_step(topk_ids=ids, topk_w=tw, x=_bf16(x), w=_bf16(w), **g)
    lo = cfg.my_rank * cfg.n_experts_local
    seen = 0
    for rk in range(cfg.n_ranks):
        buf = res["recv_bufs"][rk].reshape(cfg.tokens_per_rank, cfg.top_k, cfg.msg + pad)
        for t in range(cfg.tokens_per_rank):
            for k in range(cfg.top_k):
                slot = buf[t, k]
                gexp = int(ids[rk, t, k])
                if lo <= gexp < lo + cfg.n_experts_local:
                    row = O.bf16_to_f64(slot[: 2 * cfg.n].view("<u2"))
                    assert row[:4].tolist() == [rk + 1, t + 1, k + 1, gexp - lo + 1]
                    assert np.all(row[4:] == 0)
                    assert np.all(slot[2 * cfg.n:] == 0xFF)
                    seen += 1
                else:
                    assert np.all(slot == 0xFF)
    assert seen == M
    assert res["err"] == 0


def test_counts_match_histogram():
    cfg = TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4, tokens_per_rank=64, top_k=4, seed=3)
    ids, _ = make_routing(cfg)
    off, _ = O.group_local_picks(ids, 4, 0)
    words = O.recv_counts(off, 4, 4)
    hist = Counter()
    for rk in range(4):
        for t in range(64):
            for k in range(4):
                if ids[rk, t, k] < 4:
                    hist[(int(ids[rk, t, k]), rk)] += 1
    for e in range(4):
        for rk in range(4):
            assert words[e * 4 + rk] == hist[(e, rk)]
    assert words.sum() == off[-1]


@pytest.mark.parametrize("R,El", [(1, 1), (2, 3), (3, 2)])
def test_election_sets_flag_only_after_all_experts(R, El):
    """Every total order of the E_l*R signals: rank rk's flag flips exactly at
    the E_l-th signal for rk, and by then all of rk's count words are final."""
    sig = [(e, rk) for e in range(El) for rk in range(R)]
    orders = itertools.permutations(sig) if len(sig) <= 6 else \
        (np.random.default_rng(0).permutation(sig).tolist() for _ in range(200))
    for order in orders:
        model = O.ElectionModel(R, El, epoch=5)
        done = Counter()
        for e, rk in order:
            elected = model.signal(e, rk, 100 + e * R + rk)
            done[rk] += 1
            assert elected == (done[rk] == El)
            for r in range(R):
                assert (model.flag(r) == 5) == (done[r] == El)
            if elected:
                for ee in range(El):
                    assert model.words[O.recv_count_index(ee, rk, R)] == 100 + ee * R + rk
        assert np.all(model.counter == 0)


def test_final_control_matches_model():
    cfg = TINY.replace(seed=4)
    ids, _ = make_routing(cfg)
    off, _ = O.group_local_picks(ids, cfg.n_experts_local, 0)
    model = O.ElectionModel(cfg.n_ranks, cfg.n_experts_local, epoch=3)
    for e in range(cfg.n_experts_local):
        for rk in range(cfg.n_ranks):
            model.signal(e, rk, off[e * cfg.n_ranks + rk + 1] - off[e * cfg.n_ranks + rk])
    ctrl = O.final_control(off, cfg.n_ranks, cfg.n_experts_local, 3)
    assert np.array_equal(ctrl["words"], model.words)


def test_one_hot_weights_return_the_slot():
    inp = make_inputs(TINY)
    tw = np.zeros_like(inp.topk_w)
    lo, El = 0, TINY.n_experts_local
    for rk in range(TINY.n_ranks):
        for t in range(TINY.tokens_per_rank):
            loc = [k for k in range(TINY.top_k) if lo <= inp.topk_ids[rk, t, k] < lo + El]
            if loc:
                tw[rk, t, loc[0]] = 1.0
    res = O.run_step(topk_ids=inp.topk_ids, topk_w=tw, x_rows=inp.rows, w=inp.w, **_geom(TINY))
    for rk in range(TINY.n_ranks):
        for t in range(TINY.tokens_per_rank):
            loc = [k for k in range(TINY.top_k) if lo <= inp.topk_ids[rk, t, k] < lo + El]
            got = res["out_bits"][rk, t]
            if loc:
                off = O.recv_slot_offset(t, loc[0], 0, TINY.top_k, TINY.msg)
                assert np.array_equal(got, res["recv_bufs"][rk][off:off + 2 * TINY.n].view("<u2"))
            else:
                assert np.all(got == 0)


def _brute_y(x, w, e):
    xr = O.bf16_to_f64(x)
    we = O.bf16_to_f64(w[e])
    return [sum(float(xr[k]) * float(we[n][k]) for k in range(len(xr))) for n in range(we.shape[0])]


def test_partial_combines_sum_to_full_moe_combine():
    """Summing the per-share combines of every my_rank gives the whole MoE
    combine sum_k w_k * y_(t,k), computed here by brute force over all picks.
    Inputs are small integers and weights are sums of a few powers of two, so
    every product and sum on both sides is exact and the results must agree
    bit for bit: any pick counted twice, dropped, or sent to the wrong share
    shows."""
    R, Eg, T, k, K, N = 2, 4, 3, 2, 12, 8
    El = Eg // R
    rng = np.random.default_rng(7)
    ids = np.stack([np.stack([rng.permutation(Eg)[:k] for _ in range(T)]) for _ in range(R)]).astype(np.int32)
    tw = (rng.integers(1, 8, (R, T, k)) / 8.0).astype(np.float32)
    W = _bf16(rng.integers(-2, 3, (Eg, N, K)))            # all global experts
    Xtok = _bf16(rng.integers(-2, 3, (R, T, k, K)))       # one input row per pick
    total = np.zeros((R, T, N))
    for my in range(R):
        off, src = O.group_local_picks(ids, El, my)
        M = int(off[-1])
        x = np.zeros((M, K), np.uint16)
        for m in range(M):
            _, rk = O.row_owner(off, R, m)
            x[m] = Xtok[rk, src[m][0], src[m][1]]
        res = O.run_step(topk_ids=ids, topk_w=tw, x=x, w=W[my * El:(my + 1) * El], n_ranks=R,
                         n_experts_per_device=El, top_k=k, msg_bytes=2 * N,
                         max_tokens_per_rank=T, my_rank=my)
        total += O.bf16_to_f64(res["out_bits"])
        # the share's own output is the combine of its own picks only
        part = np.zeros((R, T, N))
        for rk in range(R):
            for t in range(T):
                for kk in range(k):
                    if my * El <= ids[rk, t, kk] < (my + 1) * El:
                        y = np.array(_brute_y(Xtok[rk, t, kk], W, int(ids[rk, t, kk])))
                        part[rk, t] += float(tw[rk, t, kk]) * y
        assert np.array_equal(res["out_bits"], O.f64_to_bf16(part))
    full = np.zeros((R, T, N))
    for rk in range(R):
        for t in range(T):
            for kk in range(k):
                y = np.array(_brute_y(Xtok[rk, t, kk], W, int(ids[rk, t, kk])))
                full[rk, t] += float(tw[rk, t, kk]) * y
    assert np.array_equal(total, full)


def test_all_local_identity_combine_closed_form():
    """R=1 with every expert local and W=I: out = bf16(acc) with acc the
    binary32 fused multiply-add chain of w_k * x_(t,k) in ascending k (each
    step rounded exactly, by rational arithmetic)."""
    from test_oracle_combine import fmaf_exact
    cfg = TINY.replace(n_ranks=1, n_experts_global=3, n_experts_local=3, tokens_per_rank=6,
                       top_k=3, k=64, n=64)
    ids, tw = make_routing(cfg)
    off, src = O.group_local_picks(ids, 3, 0)
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((int(off[-1]), 64)))
    w = _bf16(np.stack([np.eye(64)] * 3))
    res = O.run_step(topk_ids=ids, topk_w=tw, x=x, w=w, **_geom(cfg))
    for t in range(6):
        acc = [0.0] * 64
        for kk in range(3):
            m = next(m for m in range(int(off[-1])) if tuple(src[m]) == (t, kk))
            xv = O.bf16_to_f64(x[m])
            acc = [fmaf_exact(float(tw[0, t, kk]), float(xv[j]), acc[j]) for j in range(64)]
        assert np.array_equal(res["out_bits"][0, t], O.f64_to_bf16(np.array(acc)))


def test_out_of_range_slot_is_rejected_and_untouched():
    cfg = TINY
    inp = make_inputs(cfg)
    off, src = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, 0)
    x, _ = inp.rows(O.row_picks(off, src, cfg.n_ranks))
    y_bits = O.f64_to_bf16(O.expert_rows_bf16(x, inp.w, off, cfg.n_ranks).astype(np.float64))
    bad = src.copy()
    bad[0, 0] = cfg.tokens_per_rank          # token index past max_tokens_per_rank
    bad[1, 1] = cfg.top_k                    # pick index past top_k
    recv = [np.full(cfg.tokens_per_rank * cfg.top_k * cfg.msg, 0xFF, np.uint8) for _ in range(cfg.n_ranks)]
    err = O.scatter_rows(y_bits, np.arange(2), off, bad, recv, n_ranks=cfg.n_ranks, top_k=cfg.top_k,
                         msg_bytes=cfg.msg, max_tokens_per_rank=cfg.tokens_per_rank)
    assert err == O.ORACLE_ERR_SLOT_OOB
    assert all(np.all(b == 0xFF) for b in recv)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rows_by_pick_match_rows_given_in_order(dtype):
    """Asking for X rows by pick gives the same step as passing them in the
    grouping's order (the oracle's own grouping picks the rows either way)."""
    cfg = TINY.replace(n_ranks=3, n_experts_global=9, n_experts_local=3, tokens_per_rank=40,
                       top_k=3, k=256, n=256, my_rank=1, dtype=dtype, seed=21)
    inp = make_inputs(cfg)
    g = _geom(cfg)
    a = O.run_step(topk_ids=inp.topk_ids, topk_w=inp.topk_w, x_rows=inp.rows, w=inp.w,
                   dtype=dtype, w_scale=inp.w_scale, **g)
    x, xs = inp.rows(O.row_picks(a["offsets"], a["src_info"], cfg.n_ranks))
    b = O.run_step(topk_ids=inp.topk_ids, topk_w=inp.topk_w, x=x, x_scale=xs, w=inp.w,
                   dtype=dtype, w_scale=inp.w_scale, **g)
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert all(np.array_equal(p, q) for p, q in zip(a["recv_bufs"], b["recv_bufs"]))


def test_per_expert_control_tags_every_count_word():
    # brute-force (e, rk) histogram of the local picks, independent of the
    # grouping code; the tag keeps only the low 32 bits of the epoch
    cfg = TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4, tokens_per_rank=40,
                       top_k=3, my_rank=2, seed=31)
    inp = make_inputs(cfg)
    R, El = cfg.n_ranks, cfg.n_experts_local
    hist = np.zeros((El, R), dtype=np.int64)
    for rk in range(R):
        for t in range(cfg.tokens_per_rank):
            for k in range(cfg.top_k):
                g = int(inp.topk_ids[rk, t, k]) - cfg.my_rank * El
                if 0 <= g < El:
                    hist[g, rk] += 1
    epoch = (7 << 32) + 123
    off, _ = O.group_local_picks(inp.topk_ids, El, cfg.my_rank)
    ctrl = O.final_control_per_expert(off, R, El, epoch)
    words = ctrl["words"]
    for e in range(El):
        for rk in range(R):
            w = int(words[e * R + rk])
            assert w & 0xFFFFFFFF == hist[e, rk]
            assert w >> 32 == 123
    assert np.all(words[El * R:] == 0)
    # the rank-level control differs only in the tags and the flags
    lvl = O.final_control(off, R, El, epoch)["words"]
    assert np.array_equal(words[:El * R] & np.uint64(0xFFFFFFFF), lvl[:El * R])

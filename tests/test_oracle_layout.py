"""Pins of the oracle's index formulas and grouping: a hand-derived worked
example, library routines for row-major indexing, and pure-Python brute force."""
import itertools
import json
import os
from collections import Counter

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_recv_count_index_is_row_major():
    for El, R in [(1, 1), (2, 2), (32, 8), (16, 8), (5, 3)]:
        e, rk = np.meshgrid(np.arange(El), np.arange(R), indexing="ij")
        got = O.recv_count_index(e, rk, R)
        assert np.array_equal(got, np.ravel_multi_index((e, rk), (El, R)))
        assert sorted(got.ravel().tolist()) == list(range(El * R))


def test_recv_slot_offsets_tile_the_buffer():
    for T, k, msg in [(8, 2, 256), (5, 3, 48), (128, 8, 14336)]:
        t, kk = np.meshgrid(np.arange(T), np.arange(k), indexing="ij")
        off = O.recv_slot_offset(t, kk, 0, k, msg)
        assert np.array_equal(off, np.ravel_multi_index((t, kk), (T, k)) * msg)
        starts = np.sort(off.ravel())
        assert starts[0] == 0 and np.all(np.diff(starts) == msg)
        assert starts[-1] + msg == T * k * msg
        # byte_off moves within the message
        assert O.recv_slot_offset(3 % T, 1 % k, 7, k, msg) == O.recv_slot_offset(3 % T, 1 % k, 0, k, msg) + 7


def test_worked_example_grouping_counts_slots():
    g = _golden()
    ids = np.array(g["topk_ids"], dtype=np.int32)
    offsets, src = O.group_local_picks(ids, g["n_experts_per_device"], g["my_rank"])
    assert offsets.tolist() == g["offsets"]
    assert src.tolist() == g["src_info"]
    R = g["n_ranks"]
    assert O.recv_counts(offsets, R, g["n_experts_per_device"]).tolist() == g["recv_count_words"]
    for m, (rk, off) in enumerate(g["slot_rank_and_byte_offset"]):
        e, r = O.row_owner(offsets, R, m)
        t, k = src[m]
        assert r == rk
        assert O.recv_slot_offset(int(t), int(k), 0, g["top_k"], g["msg_bytes"]) == off


def test_worked_example_full_step():
    g = _golden()
    ids = np.array(g["topk_ids"], dtype=np.int32)
    tw = np.array(g["topk_w"], dtype=np.float32)
    K, N, El = g["k"], g["n"], g["n_experts_per_device"]
    M = g["offsets"][-1]
    xf = np.zeros((M, K), dtype=np.float32)
    xf[:, 0] = np.arange(1, M + 1)
    wf = np.stack([np.eye(N, K), 2 * np.eye(N, K)]).astype(np.float32)
    import torch
    xb = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wb = torch.from_numpy(wf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    res = O.run_step(topk_ids=ids, topk_w=tw, x=xb, w=wb, n_ranks=g["n_ranks"],
                     n_experts_per_device=El, top_k=g["top_k"], msg_bytes=g["msg_bytes"],
                     max_tokens_per_rank=g["tokens_per_rank"], my_rank=g["my_rank"], epoch=7)
    out = O.bf16_to_f64(res["out_bits"])
    assert out[..., 0].tolist() == g["combine_first_column"]
    assert np.all(out[..., 1:] == 0)
    for rk, off in g["untouched_slots_rank_and_byte_offset"]:
        assert np.all(res["recv_bufs"][rk][off:off + g["msg_bytes"]] == 0xFF)
    w = res["control"]["words"]
    assert w[:El * g["n_ranks"]].tolist() == g["recv_count_words"]
    assert w[El * g["n_ranks"]:].tolist() == [7, 7]


def _brute_group(ids, El, my_rank):
    R, T, K = ids.shape
    rows = []
    for rk in range(R):
        for t in range(T):
            for k in range(K):
                gexp = int(ids[rk][t][k])
                if my_rank * El <= gexp < (my_rank + 1) * El:
                    rows.append((gexp - my_rank * El, rk, t, k))
    rows.sort()
    offsets = [0]
    for e in range(El):
        for rk in range(R):
            offsets.append(offsets[-1] + sum(1 for r in rows if r[0] == e and r[1] == rk))
    return offsets, [(r[2], r[3]) for r in rows]


@pytest.mark.parametrize("seed", range(12))
def test_grouping_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.integers(1, 9))
    Eg = int(rng.integers(1, 5)) * R
    El = Eg // R
    T = int(rng.integers(1, 9))
    k = int(rng.integers(1, Eg + 1))
    my_rank = int(rng.integers(0, R))
    ids = np.stack([np.stack([rng.permutation(Eg)[:k] for _ in range(T)]) for _ in range(R)]).astype(np.int32)
    off, src = O.group_local_picks(ids, El, my_rank)
    boff, bsrc = _brute_group(ids, El, my_rank)
    assert off.tolist() == boff
    assert [tuple(s) for s in src.tolist()] == bsrc
    # invariants: monotone offsets, every local pick exactly once
    assert np.all(np.diff(off) >= 0)
    picks = Counter()
    for m, (t, kk) in enumerate(src.tolist()):
        e, rk = O.row_owner(off, R, m)
        assert int(ids[rk, t, kk]) == my_rank * El + e
        picks[(rk, t, kk)] += 1
    assert all(v == 1 for v in picks.values())
    assert len(picks) == sum(1 for rk, t, kk in itertools.product(range(R), range(T), range(k))
                             if my_rank * El <= ids[rk, t, kk] < (my_rank + 1) * El)


@pytest.mark.parametrize("seed", range(4))
def test_row_picks_name_each_local_pick_once(seed):
    """row_picks: the pick (rk, t, k) of every grouped row routes to the row's
    own expert, and the picks of all rows are exactly the local picks (a brute
    force over the routing)."""
    rng = np.random.default_rng(200 + seed)
    R, El, T, k = int(rng.integers(1, 6)), int(rng.integers(1, 5)), int(rng.integers(1, 30)), 3
    my = int(rng.integers(0, R))
    Eg = max(R * El, k)
    ids = np.stack([np.stack([rng.permutation(Eg)[:k] for _ in range(T)])
                    for _ in range(R)]).astype(np.int32)
    off, src = O.group_local_picks(ids, El, my)
    picks = O.row_picks(off, src, R)
    lo = my * El
    for m, (rk, t, kk) in enumerate(picks.tolist()):
        e = next(e for e in range(El) if off[e * R] <= m < off[(e + 1) * R])
        assert ids[rk, t, kk] == lo + e
    want = sorted((rk, t, kk) for rk in range(R) for t in range(T) for kk in range(k)
                  if lo <= ids[rk, t, kk] < lo + El)
    assert sorted(map(tuple, picks.tolist())) == want


def test_dispatch_rows_give_each_row_its_tokens_row():
    """dispatch_rows: by brute force over the routing, the row of every local
    pick (rk, t, k) is token t of rank rk, whatever k, in grouped order."""
    rng = np.random.default_rng(300)
    R, El, T, k, H = 3, 2, 7, 3, 5
    ids = np.stack([np.stack([rng.permutation(R * El)[:k] for _ in range(T)])
                    for _ in range(R)]).astype(np.int32)
    toks = rng.integers(0, 1000, (R, T, H))
    for my in range(R):
        off, src = O.group_local_picks(ids, El, my)
        x = O.dispatch_rows(toks, off, src, R)
        want = []
        for e in range(El):
            for rk in range(R):
                for t in range(T):
                    for kk in range(k):
                        if ids[rk, t, kk] == my * El + e:
                            want.append(toks[rk, t])
        assert np.array_equal(x, np.array(want).reshape(-1, H))

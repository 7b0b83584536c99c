"""Balanced row tiles of the bf16 256-column tile (up to 288 rows) through the
C ABI, on a routing built so that the local experts hold exactly the group
sizes at the tiling's edges: one row, a block and a row, 256, 257 (nine
blocks, the last with one row), 288 (nine full blocks), 289 (two tiles of
five blocks), 576 and 577 (two and three tiles), 1030 (four tiles, one of
nine blocks) and an empty expert.  Values against the oracle, as in the named
parity cases; the tile trace must split each expert's 32-row blocks as the
tiling prescribes: with B = ceil(M_e / 32) and mt = ceil(B / 9) tiles, tile
mb takes blocks [mb * B / mt, (mb + 1) * B / mt)."""
import numpy as np
import pytest
import torch

from ep_synth import TINY, make_inputs

SIZES = [288, 289, 256, 257, 1, 33, 32, 576, 577, 0, 1030, 100]
CFG = TINY.replace(n_ranks=2, n_experts_global=24, n_experts_local=len(SIZES),
                   tokens_per_rank=1024, top_k=2, k=128, n=512, seed=41)


def routing(sizes, cfg):
    """Routing ids [R][T][2] whose local picks give expert e exactly sizes[e]
    rows: pick 0 of every token, then pick 1 of the first tokens, take the
    local experts in ascending order (a token's two picks then differ, every
    expert having at most R*T picks); the other picks go to remote experts."""
    R, T, El = cfg.n_ranks, cfg.tokens_per_rank, cfg.n_experts_local
    assert cfg.top_k == 2 and max(sizes) <= R * T and sum(sizes) <= 2 * R * T
    local = np.repeat(np.arange(El), sizes)
    ids = np.empty((R * T, 2), dtype=np.int32)
    ids[:, 0] = local[: R * T]
    rest = local[R * T:]
    ids[: len(rest), 1] = rest
    i = np.arange(len(rest), R * T)
    ids[len(rest):, 1] = El + i % El              # remote experts
    return ids.reshape(R, T, 2)


def expected_tiles(m):
    """(first row, rows) of each row tile of an expert of m rows."""
    if m == 0:
        return []
    b = (m + 31) // 32
    mt = (b + 8) // 9
    out = []
    for mb in range(mt):
        b0, b1 = mb * b // mt, (mb + 1) * b // mt
        out.append((32 * b0, min(32 * b1, m) - 32 * b0))
    return out


def test_routing_gives_the_sizes():
    """CPU: the constructed routing has exactly the intended group sizes and
    no token picks one expert twice."""
    import oracle as O
    ids = routing(SIZES, CFG)
    off, _ = O.group_local_picks(ids, CFG.n_experts_local, CFG.my_rank)
    assert list(np.diff(off[:: CFG.n_ranks])) == SIZES
    assert np.all(ids[..., 0] != ids[..., 1])
    # the tiling's edges: nine-block tiles, a one-row last block, several tiles
    tiles = {m: expected_tiles(m) for m in SIZES}
    assert tiles[288] == [(0, 288)] and tiles[257] == [(0, 257)]
    assert tiles[289] == [(0, 160), (160, 129)] and len(tiles[577]) == 3
    assert [r for _, r in tiles[1030]] == [256, 256, 256, 262]


@pytest.mark.gpu
def test_balanced_row_tiles_match_the_oracle_and_the_tiling():
    from gpu_helpers import compare_step, device_inputs, make_ctx, oracle_step
    cfg = CFG
    print(f"[case] row tiles {SIZES}", flush=True)
    inp = make_inputs(cfg)
    ids = routing(SIZES, cfg)
    ctx = make_ctx(cfg, trace_records=4096)
    assert ctx.gemm_tile(sum(SIZES)) == (0, 288, 256)
    d = device_inputs(inp, ctx, topk_ids=ids)
    assert d["m_total"] == sum(SIZES)
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    ctx.reset_trace()
    ctx.step(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"], d["topk_ids"],
             d["topk_w"], out)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    ref = oracle_step(inp, epoch=ctx.epoch, topk_ids=ids)
    compare_step(ctx, ref, cfg, out, cfg.msg, ctx.epoch)

    tab = ctx.trace_table()
    off = ref["offsets"]
    R = cfg.n_ranks
    for e, m in enumerate(SIZES):
        g0 = int(off[e * R])
        sel = tab["expert"] == e
        for n0 in range(0, cfg.n, 256):
            got = sorted((int(m0) - g0, int(r)) for m0, r in
                         zip(tab["m0"][sel & (tab["n0"] == n0)], tab["rows"][sel & (tab["n0"] == n0)]))
            assert got == expected_tiles(m), (e, m, n0, got)
        assert np.all(tab["cols"][sel] == 256)

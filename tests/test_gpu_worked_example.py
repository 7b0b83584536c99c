"""The hand-derived worked example (tests/golden/worked_example.json) through
the whole HIP path: grouping, grouped GEMM with the scatter epilogue, count
words, and the combine, checked against the example's own numbers rather than
against the oracle.  The kernels take K in multiples of 64 and N in multiples
of 128, so the example's 8 x 8 problem is embedded at K = 64, N = 128 with
zero padding (identity weights keep every value exact); slot byte offsets
scale with the 256-byte slots."""
import json
from pathlib import Path

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

G = json.loads((Path(__file__).parent / "golden" / "worked_example.json").read_text())
K, N = 64, 128
MSG = 2 * N


def test_worked_example_through_the_hip_path():
    from grouped_gemm_scatter_amd import EpCombine
    R, El, T, k = G["n_ranks"], G["n_experts_per_device"], G["tokens_per_rank"], G["top_k"]
    ctx = EpCombine(n_ranks=R, top_k=k, max_tokens_per_rank=T, n_experts_per_device=El,
                    hidden_k=K, hidden_n=N, my_rank=G["my_rank"], msg_bytes=MSG, sentinel=0xFF)
    ids = torch.tensor(G["topk_ids"], dtype=torch.int32, device="cuda")
    tw = torch.tensor(G["topk_w"], dtype=torch.float32, device="cuda")
    off, src = ctx.group(ids)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == G["offsets"]
    M = G["offsets"][-1]
    assert src[:M].cpu().tolist() == G["src_info"]

    # x row m = (m + 1) * e_0; W_0 = identity, W_1 = 2 * identity (stored [E_l][N][K])
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    x[:, 0] = torch.arange(1, M + 1, dtype=torch.float32, device="cuda").to(torch.bfloat16)
    w = torch.zeros((El, N, K), dtype=torch.bfloat16, device="cuda")
    for e in range(El):
        w[e, :K, :K] = (e + 1) * torch.eye(K, dtype=torch.bfloat16, device="cuda")
    out = torch.empty((R, T, N), dtype=torch.bfloat16, device="cuda")
    ctx.step(x, w, off, src, M, ids, tw, out)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0

    assert ctx.counts.cpu().tolist() == G["recv_count_words"]
    assert ctx.flags.cpu().tolist() == [ctx.epoch] * R
    # each row at its slot: first column (m + 1) for expert 0 rows, 2 (m + 1) for expert 1
    bounds = G["offsets"]
    for m, (rk, off16) in enumerate(G["slot_rank_and_byte_offset"]):
        e = 0 if m < bounds[R] else 1
        row = ctx.recv[rk][off16 // 16 * MSG: off16 // 16 * MSG + 2 * N].cpu()
        vals = row.view(torch.bfloat16).float()
        assert vals[0].item() == (e + 1) * (m + 1), (m, vals[0].item())
        assert torch.all(vals[1:] == 0)
    for rk, off16 in G["untouched_slots_rank_and_byte_offset"]:
        assert torch.all(ctx.recv[rk][off16 // 16 * MSG: off16 // 16 * MSG + MSG] == 0xFF)
    o = out.float().cpu()
    assert o[..., 0].tolist() == G["combine_first_column"]
    assert torch.all(o[..., 1:] == 0)

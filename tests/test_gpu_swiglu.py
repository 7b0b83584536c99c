"""GPU parity of the up-projection with SwiGLU (ep_grouped_gemm_swiglu, the
expert FFN's first GEMM feeding the down-projection's X): every output element
against the oracle on small shapes (several tiles, ragged group tails, empty
experts, several ranks) and at the full benchmark shapes, and the guard rows
around the output left untouched.  The HIP side groups the routing itself
(ep_group_local_picks); the oracle derives its own grouping; X1 rows come
from the generator per pick."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import CONFIGS, TINY, make_inputs

pytestmark = pytest.mark.gpu

from gpu_helpers import BF16_TOL, assert_close, layout_picks, make_ctx  # noqa: E402

GUARD = 0x5A5A

CASES = {
    # hidden = n (K of this GEMM), I = k (its output width)
    "two_tiles_ragged": TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4,
                                     tokens_per_rank=300, top_k=4, k=128, n=256, my_rank=1,
                                     seed=31),
    "wide_output": TINY.replace(n_ranks=3, n_experts_global=9, n_experts_local=3,
                                tokens_per_rank=200, top_k=3, k=384, n=384, my_rank=2, seed=32),
    "zipf_empty_experts": TINY.replace(n_ranks=8, n_experts_global=64, n_experts_local=8,
                                       tokens_per_rank=256, top_k=6, k=256, n=384,
                                       routing="zipf", n_forced_empty=2, seed=33),
}


def _run(cfg):
    inp = make_inputs(cfg)
    I = cfg.k
    ctx = make_ctx(cfg)
    offsets, src_info = ctx.group(torch.from_numpy(inp.topk_ids.astype(np.int32)).cuda())
    M = int(offsets[-1].item())
    x1 = inp.up_rows(layout_picks(offsets, src_info, cfg.n_ranks, M))
    w1 = inp.up_weights()
    out = torch.full((M + 2, I), 0, dtype=torch.int16, device="cuda").fill_(GUARD)
    h = out.view(torch.bfloat16)[1:M + 1]
    ctx.up_swiglu(torch.from_numpy(x1).view(torch.bfloat16).cuda() if M else None,
                  torch.from_numpy(w1).view(torch.bfloat16).cuda(), offsets, M, h if M else None)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    got = out.cpu().numpy().view(np.uint16)
    assert np.all(got[0] == GUARD) and np.all(got[M + 1] == GUARD), "guard rows touched"
    # the oracle: its own grouping, the rows of its own picks
    off_o, src_o = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    x1_o = inp.up_rows(O.row_picks(off_o, src_o, cfg.n_ranks))
    ref = O.f64_to_bf16(O.expert_swiglu(x1_o, w1, off_o, cfg.n_ranks).astype(np.float64))
    return got[1:M + 1], ref


@pytest.mark.parametrize("name", sorted(CASES))
def test_swiglu_matches_oracle(name):
    cfg = CASES[name]
    print(f"[case] swiglu {cfg}", flush=True)
    got, ref = _run(cfg)
    assert_close(got, ref, BF16_TOL, f"{name} h")


@pytest.mark.parametrize("name", ["deepseek_prefill", "qwen3_moe"])
def test_swiglu_full_size(name):
    cfg = CONFIGS[name]
    print(f"[case] swiglu full size {name}", flush=True)
    got, ref = _run(cfg)
    assert_close(got, ref, BF16_TOL, f"{name} h")


def test_swiglu_rejects_fp8_handles_and_unaligned_widths():
    from grouped_gemm_scatter_amd import EP_ERR_UNSUPPORTED, EpError
    cfg = CASES["two_tiles_ragged"]
    # sized for the wider of the two handles, so that only the library's own
    # check can reject the call
    w1 = torch.zeros((cfg.n_experts_local, 2 * 192, cfg.n), dtype=torch.bfloat16, device="cuda")
    off = torch.zeros(cfg.n_experts_local * cfg.n_ranks + 1, dtype=torch.int32, device="cuda")
    for bad in [cfg.replace(dtype="fp8"), cfg.replace(k=192)]:
        ctx = make_ctx(bad)
        with pytest.raises(EpError) as ei:
            ctx.up_swiglu(None, w1, off, 0, None)
        assert ei.value.code == EP_ERR_UNSUPPORTED

"""The allocation-free GEMM entry point (ep_grouped_gemm_scatter_noalloc)
against ep_grouped_gemm_scatter on the same inputs: two calls in a row, the
second on a smaller input, each followed by the combine.  The two share their
kernels, so receive buffers, control words and combined outputs must agree
bit for bit; the handle's own counters stay untouched by the allocation-free
form, and its library-held counters end each step re-armed (the next call's
elections complete)."""
import numpy as np
import pytest
import torch

from ep_synth import TINY, make_inputs
from gpu_helpers import bits, device_inputs, make_ctx

pytestmark = pytest.mark.gpu

BIG = TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4, tokens_per_rank=384,
                   top_k=4, k=512, n=512, my_rank=1, seed=41)
SMALL = TINY.replace(n_ranks=4, n_experts_global=16, n_experts_local=4, tokens_per_rank=40,
                     top_k=4, k=512, n=512, my_rank=1, seed=42)


def test_noalloc_matches_the_allocating_entry_point():
    T_max = BIG.tokens_per_rank
    ref = make_ctx(BIG, max_tokens=T_max)       # ep_grouped_gemm_scatter
    na = make_ctx(BIG, max_tokens=T_max)        # ep_grouped_gemm_scatter_noalloc
    for cfg in (BIG, SMALL):
        print(f"[case] noalloc {cfg}", flush=True)
        inp = make_inputs(cfg)
        d = device_inputs(inp, ref)
        outs = []
        for ctx, noalloc in ((ref, False), (na, True)):
            out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                             dtype=torch.bfloat16, device="cuda")
            ctx.next_epoch()
            ctx.gemm_scatter(d["x"], d["w"], d["offsets"], d["src_info"], d["m_total"],
                             noalloc=noalloc)
            ctx.combine(d["topk_ids"], d["topk_w"], out)
            torch.cuda.synchronize()
            assert ctx.query_error() == 0
            outs.append(out)
        assert na.epoch == ref.epoch
        for rk in range(cfg.n_ranks):
            assert torch.equal(na.recv[rk], ref.recv[rk]), f"rank {rk}: receive buffer differs"
        assert torch.equal(na.words, ref.words), "count words / flags differ"
        assert np.all(ref.flags.cpu().numpy() == ref.epoch)
        assert np.array_equal(bits(outs[1]), bits(outs[0])), "combined output differs"
        # the allocation-free form never touches the handle's own counters
        assert torch.all(na.rank_counter == 0) and torch.all(na.tile_counter == 0)
        assert torch.all(ref.rank_counter == 0) and torch.all(ref.tile_counter == 0)

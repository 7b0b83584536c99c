"""Dispatch side (ep_dispatch_rows): every grouped row receives its pick's
token row.  A byte copy, so compared bit for bit with the oracle's
dispatch_rows on the oracle's own grouping, at small shapes (several ranks,
empty experts, no local rows) and at the full prefill and Qwen3 sizes; a token
index outside the source arrays is latched and its row left unwritten."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import CONFIGS, make_inputs
from gpu_helpers import make_ctx, to_dev
from test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


def _dispatch(cfg):
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    toks = inp.tokens()
    offsets, src_info = ctx.group(to_dev(inp.topk_ids.astype(np.int32)))
    M = int(offsets[-1].item())
    x = torch.full((M + 1, cfg.n), -7.0, dtype=torch.bfloat16, device="cuda")   # + a guard row
    ctx.dispatch(to_dev(toks, torch.bfloat16), offsets, src_info, M, x)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    got = x.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(O.bf16_to_f64(got[M]) == -7.0), "the row past m_total was written"
    off_o, src_o = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    want = O.dispatch_rows(toks, off_o, src_o, cfg.n_ranks)
    assert np.array_equal(got[:M], want.reshape(M, cfg.n))


@pytest.mark.parametrize("name", ["tiny", "multi_tile_256", "zipf_empty_experts", "no_local_rows",
                                  "many_experts_ragged", "combine_rows_7680"])
def test_dispatch_matches_oracle(name):
    print(f"[case] dispatch {name}", flush=True)
    _dispatch(CASES[name])


@pytest.mark.parametrize("name", ["deepseek_prefill", "qwen3_moe"])
def test_dispatch_full_size(name):
    print(f"[case] dispatch full size {name}", flush=True)
    _dispatch(CONFIGS[name])


def test_dispatch_bad_token_index_is_latched():
    cfg = CASES["multi_tile_256"]
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    offsets, src_info = ctx.group(to_dev(inp.topk_ids.astype(np.int32)))
    M = int(offsets[-1].item())
    src_info[3, 0] = cfg.tokens_per_rank            # row 3 names a token past the arrays
    x = torch.full((M, cfg.n), -7.0, dtype=torch.bfloat16, device="cuda")
    ctx.dispatch(to_dev(inp.tokens(), torch.bfloat16), offsets, src_info, M, x)
    assert ctx.query_error() == 4                    # EP_ERR_BAD_GROUP
    assert torch.all(x[3] == -7.0) and not torch.all(x[4] == -7.0)

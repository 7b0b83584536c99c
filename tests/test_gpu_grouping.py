"""Local grouping on the GPU (ep_group_local_picks) against the oracle's
group_local_picks: offsets and src_info are integer results, compared
bit-exactly, at small shapes with empty experts, no local picks, a non-zero
rank, dropped picks (id -1) and zero tokens, and at every full workload."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import CONFIGS, make_routing
from gpu_helpers import make_ctx
from test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


def _check(cfg, ids):
    ctx = make_ctx(cfg)
    d_ids = torch.from_numpy(np.ascontiguousarray(ids.astype(np.int32))).cuda()
    off, src = ctx.group(d_ids)
    torch.cuda.synchronize()
    want_off, want_src = O.group_local_picks(ids, cfg.n_experts_local, cfg.my_rank)
    got_off = off.cpu().numpy().astype(np.int64)
    assert np.array_equal(got_off, want_off), "offsets differ"
    m = int(got_off[-1])
    assert np.array_equal(src.cpu().numpy()[:m].astype(np.int64), want_src), "src_info differs"
    return m


@pytest.mark.parametrize("name", ["tiny", "zipf_empty_experts", "no_local_rows",
                                  "many_experts_ragged", "decode_zipf_empty_experts",
                                  "split_tail_mixed"])
def test_grouping_matches_the_oracle(name):
    cfg = CASES[name]
    print(f"[case] grouping {name}", flush=True)
    ids, *_ = make_routing(cfg)
    _check(cfg, ids)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_grouping_full_size(name):
    cfg = CONFIGS[name]
    print(f"[case] grouping full size {name}", flush=True)
    ids, *_ = make_routing(cfg)
    m = _check(cfg, ids)
    assert m > 0 or name == "tiny"


def test_grouping_skips_dropped_picks_and_other_ranks_experts():
    cfg = CASES["many_experts_ragged"].replace(my_rank=3)
    print("[case] grouping dropped picks", flush=True)
    ids, *_ = make_routing(cfg)
    ids = ids.copy()
    rng = np.random.default_rng(5)
    ids[rng.random(ids.shape) < 0.2] = -1           # dropped picks are never rows
    _check(cfg, ids)


def test_grouping_of_zero_tokens():
    cfg = CASES["tiny"]
    ctx = make_ctx(cfg)
    ids = torch.empty((cfg.n_ranks, 0, cfg.top_k), dtype=torch.int32, device="cuda")
    off, _ = ctx.group(ids)
    torch.cuda.synchronize()
    assert torch.all(off == 0)

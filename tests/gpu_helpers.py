"""Helpers for the GPU parity tests: run one step through the C ABI on seeded
inputs and compare every output with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

BF16_TOL = 2e-2      # |gpu - oracle| <= tol * max(1, |oracle|), bf16 inputs
FP8_TOL = 5e-2       # same, fp8 inputs
SENTINEL = 0xFF


def tol_for(cfg):
    return FP8_TOL if cfg.dtype == "fp8" else BF16_TOL


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def device_inputs(inp):
    """Copies the generator's arrays to the GPU with the dtypes the ABI expects."""
    fp8 = inp.cfg.dtype == "fp8"
    d = {
        "x": to_dev(inp.x, torch.uint8 if fp8 else torch.bfloat16),
        "w": to_dev(inp.w, torch.uint8 if fp8 else torch.bfloat16),
        "offsets": to_dev(inp.offsets.astype(np.int32)),
        "src_info": to_dev(inp.src_info.astype(np.int32)),
        "topk_ids": to_dev(inp.topk_ids.astype(np.int32)),
        "topk_w": to_dev(inp.topk_w.astype(np.float32)),
        "x_scale": to_dev(inp.x_scale) if fp8 else None,
        "w_scale": to_dev(inp.w_scale) if fp8 else None,
    }
    if d["x"].dim() == 2 and d["x"].shape[0] == 0:
        d["x"] = None
    return d


def make_ctx(cfg, msg_bytes=None, **kw):
    from grouped_gemm_scatter_amd import EpCombine
    return EpCombine(n_ranks=cfg.n_ranks, top_k=cfg.top_k,
                     max_tokens_per_rank=cfg.tokens_per_rank,
                     n_experts_per_device=cfg.n_experts_local, hidden_k=cfg.k, hidden_n=cfg.n,
                     my_rank=cfg.my_rank, msg_bytes=msg_bytes or cfg.msg, dtype=cfg.dtype,
                     sentinel=SENTINEL, **kw)


def oracle_step(inp, msg_bytes=None, epoch=1, per_expert=False):
    cfg = inp.cfg
    return O.run_step(topk_ids=inp.topk_ids, topk_w=inp.topk_w, x=inp.x, w=inp.w,
                      n_ranks=cfg.n_ranks, n_experts_per_device=cfg.n_experts_local,
                      top_k=cfg.top_k, msg_bytes=msg_bytes or cfg.msg,
                      max_tokens_per_rank=cfg.tokens_per_rank, my_rank=cfg.my_rank,
                      dtype=cfg.dtype, x_scale=inp.x_scale, w_scale=inp.w_scale, epoch=epoch,
                      per_expert=per_expert)


def written_mask(ref, cfg, msg_bytes):
    """Byte mask of every receive buffer: True where a local row is sent."""
    cap = cfg.tokens_per_rank * cfg.top_k * msg_bytes
    masks = [np.zeros(cap, dtype=bool) for _ in range(cfg.n_ranks)]
    off, src = ref["offsets"], ref["src_info"]
    for m in range(int(off[-1])):
        _, rk = O.row_owner(off, cfg.n_ranks, m)
        o = O.recv_slot_offset(int(src[m][0]), int(src[m][1]), 0, cfg.top_k, msg_bytes)
        masks[rk][o:o + 2 * cfg.n] = True
    return masks


def assert_close(gpu_bits, ref_bits, tol, what):
    g = O.bf16_to_f64(gpu_bits)
    r = O.bf16_to_f64(ref_bits)
    bound = tol * np.maximum(1.0, np.abs(r))
    bad = ~(np.abs(g - r) <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} values out of tolerance; "
                             f"first at {idx.tolist()}: gpu={g[bad][:5]} oracle={r[bad][:5]}")


def compare_step(ctx, ref, cfg, out, msg_bytes, epoch):
    """Bit-exact placement, counts, flags and counters; values within tolerance."""
    tol = tol_for(cfg)
    masks = written_mask(ref, cfg, msg_bytes)
    for rk in range(cfg.n_ranks):
        got = ctx.recv[rk].cpu().numpy()
        m = masks[rk]
        untouched = got[~m]
        assert np.all(untouched == SENTINEL), f"rank {rk}: bytes outside sent slots changed"
        if m.any():
            assert_close(got[m].view("<u2"), ref["recv_bufs"][rk][m].view("<u2"), tol,
                         f"rank {rk} slots")
    words = ctx.words.cpu().numpy().view(np.uint64)
    assert np.array_equal(words, ref["control"]["words"]), "count words / flags differ"
    assert np.all(ctx.rank_counter.cpu().numpy() == 0)
    assert np.all(ctx.tile_counter.cpu().numpy() == 0)
    assert_close(out.cpu().view(torch.int16).numpy().view(np.uint16), ref["out_bits"], tol,
                 "combined output")

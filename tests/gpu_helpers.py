"""Helpers for the GPU parity tests: run one step through the C ABI on seeded
inputs and compare every output with the oracle.

The two sides group the routing independently.  The HIP side takes its
layout (offsets, src_info) from the library's own grouping call
(ep_group_local_picks) and asks the generator for the X rows of the picks
that layout lists, in its order; the oracle derives its own grouping and asks
for its own rows.  The generator returns the same bytes for the same pick."""
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


def bits(t):
    """bf16 device tensor -> uint16 codes on the host."""
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def layout_picks(offsets, src_info, n_ranks, m_total):
    """(rk, t, k) of every row of a grouped layout on the device: the run of
    offsets a row falls in names its rank; src_info holds (t, k).  This is the
    dispatch's side of the harness (it assembles X in the layout's order)."""
    if m_total == 0:
        return np.zeros((0, 3), dtype=np.int64)
    rows = torch.arange(m_total, dtype=torch.int32, device=offsets.device)
    run = torch.searchsorted(offsets, rows, right=True) - 1
    rk = (run % n_ranks).to(torch.int64)
    src = src_info[:m_total].to(torch.int64)
    return torch.stack([rk, src[:, 0], src[:, 1]], dim=1).cpu().numpy()


def device_inputs(inp, ctx, topk_ids=None):
    """Device arguments of a step: routing, weights, the HIP path's own grouped
    layout of the routing (ep_group_local_picks) and the X rows of that
    layout's picks."""
    cfg = inp.cfg
    fp8 = cfg.dtype == "fp8"
    ids_h = inp.topk_ids if topk_ids is None else topk_ids
    ids = to_dev(np.asarray(ids_h, dtype=np.int32))
    offsets, src_info = ctx.group(ids)
    m_total = int(offsets[-1].item())
    picks = layout_picks(offsets, src_info, cfg.n_ranks, m_total)
    x, xs = inp.rows(picks)
    d = {
        "x": to_dev(x, torch.uint8 if fp8 else torch.bfloat16) if m_total else None,
        "w": to_dev(inp.w, torch.uint8 if fp8 else torch.bfloat16),
        "offsets": offsets,
        "src_info": src_info,
        "m_total": m_total,
        "picks": picks,
        "x_host": x,
        "topk_ids": ids,
        "topk_w": to_dev(inp.topk_w.astype(np.float32)),
        "x_scale": to_dev(xs) if fp8 and m_total else None,
        "w_scale": to_dev(inp.w_scale) if fp8 else None,
    }
    return d


def make_ctx(cfg, msg_bytes=None, max_tokens=None, **kw):
    from grouped_gemm_scatter_amd import EpCombine
    return EpCombine(n_ranks=cfg.n_ranks, top_k=cfg.top_k,
                     max_tokens_per_rank=max_tokens or cfg.tokens_per_rank,
                     n_experts_per_device=cfg.n_experts_local, hidden_k=cfg.k, hidden_n=cfg.n,
                     my_rank=cfg.my_rank, msg_bytes=msg_bytes or cfg.msg, dtype=cfg.dtype,
                     sentinel=SENTINEL, **kw)


def oracle_step(inp, msg_bytes=None, epoch=1, per_expert=False, max_tokens=None,
                topk_ids=None, topk_w=None, w=None):
    cfg = inp.cfg
    return O.run_step(topk_ids=inp.topk_ids if topk_ids is None else topk_ids,
                      topk_w=inp.topk_w if topk_w is None else topk_w,
                      w=inp.w if w is None else w, x_rows=inp.rows,
                      n_ranks=cfg.n_ranks, n_experts_per_device=cfg.n_experts_local,
                      top_k=cfg.top_k, msg_bytes=msg_bytes or cfg.msg,
                      max_tokens_per_rank=max_tokens or cfg.tokens_per_rank, my_rank=cfg.my_rank,
                      dtype=cfg.dtype, w_scale=inp.w_scale, epoch=epoch, per_expert=per_expert)


def assert_close(gpu_bits, ref_bits, tol, what, chunk=1 << 24):
    """|gpu - oracle| <= tol * max(1, |oracle|) for every bf16 value (chunked,
    so full-size arrays fit)."""
    g_all = np.asarray(gpu_bits).reshape(-1)
    r_all = np.asarray(ref_bits).reshape(-1)
    assert g_all.size == r_all.size, f"{what}: {g_all.size} values vs {r_all.size}"
    for c0 in range(0, g_all.size, chunk):
        g = O.bf16_to_f64(g_all[c0:c0 + chunk])
        r = O.bf16_to_f64(r_all[c0:c0 + chunk])
        bad = ~(np.abs(g - r) <= tol * np.maximum(1.0, np.abs(r)))
        if bad.any():
            idx = (np.nonzero(bad)[0][:5] + c0).tolist()
            raise AssertionError(f"{what}: {int(bad.sum())} values out of tolerance in chunk at "
                                 f"{c0}; first at flat {idx}: gpu={g[bad][:5]} oracle={r[bad][:5]}")


def slot_mask(ref, cfg, max_tokens, n_ranks):
    """Per rank, a bool [max_tokens*top_k] that marks the slots the oracle wrote."""
    picks = O.row_picks(ref["offsets"], ref["src_info"], n_ranks)
    masks = [np.zeros(max_tokens * cfg.top_k, dtype=bool) for _ in range(n_ranks)]
    for rk in range(n_ranks):
        p = picks[picks[:, 0] == rk]
        masks[rk][p[:, 1] * cfg.top_k + p[:, 2]] = True
    return masks


def compare_recv(ctx, ref, cfg, msg_bytes, max_tokens=None):
    """Every receive-buffer byte: each slot the oracle wrote holds its row
    within tolerance (padding bytes keep the sentinel); every other slot keeps
    the sentinel byte for byte."""
    T = max_tokens or cfg.tokens_per_rank
    tol = tol_for(cfg)
    masks = slot_mask(ref, cfg, T, cfg.n_ranks)
    for rk in range(cfg.n_ranks):
        got = ctx.recv[rk].cpu().numpy().reshape(T * cfg.top_k, msg_bytes)
        want = ref["recv_bufs"][rk].reshape(T * cfg.top_k, msg_bytes)
        m = masks[rk]
        assert np.all(got[~m] == SENTINEL), f"rank {rk}: a slot that is not sent changed"
        assert np.all(got[m, 2 * cfg.n:] == SENTINEL), f"rank {rk}: slot padding changed"
        if m.any():
            assert_close(got[m, : 2 * cfg.n].copy().view("<u2"),
                         want[m, : 2 * cfg.n].copy().view("<u2"), tol, f"rank {rk} slots")


def compare_control(ctx, ref):
    words = ctx.words.cpu().numpy().view(np.uint64)
    assert np.array_equal(words, ref["control"]["words"]), "count words / flags differ"
    assert np.all(ctx.rank_counter.cpu().numpy() == 0)
    assert np.all(ctx.tile_counter.cpu().numpy() == 0)


def compare_out(out, ref, cfg, what="combined output"):
    """Combined output within tolerance; a token with no local pick is +0,
    compared bit for bit (sign included)."""
    got = bits(out)
    assert_close(got, ref["out_bits"], tol_for(cfg), what)
    ids = np.asarray(ref["topk_ids"])
    lo = cfg.my_rank * cfg.n_experts_local
    none_local = ~((ids >= lo) & (ids < lo + cfg.n_experts_local)).any(axis=2)
    if none_local.any():
        assert np.all(got[none_local] == 0), f"{what}: a token without local picks is not +0"
        assert np.all(ref["out_bits"][none_local] == 0)


def compare_step(ctx, ref, cfg, out, msg_bytes, epoch=None, max_tokens=None):
    """Bit-exact placement, counts, flags and counters; values within tolerance."""
    compare_recv(ctx, ref, cfg, msg_bytes, max_tokens)
    compare_control(ctx, ref)
    compare_out(out, ref, cfg)

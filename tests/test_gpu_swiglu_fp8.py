"""The fp8 up-projection with SwiGLU (ep_grouped_gemm_swiglu_fp8) through the
C ABI against the oracle (expert_swiglu_fp8, then quantize_rows_e4m3).  Both
sides quantise a binary32 h in the same way, but their h differ by the
rounding of two binary32 summation orders (and the exponential), so near
small values, where the e4m3fn steps are finest, a code may differ by a few
steps: every dequantised GPU value must lie within half a quantisation step
plus the binary32 inner-product bound (gamma_n * sum |x w|, carried through
silu(g) * u) of the oracle's h, nearly all codes must be equal, and the
scales agree to the same bound.  Where h is exact on both sides (gate
sums large enough that silu(g) = g in binary32, small integer operands) codes
and scales must agree bit for bit, which checks the GPU's quantiser itself.
Then the fp8 expert FFN end to end: tokens -> dispatch (codes and scales) ->
fp8 up-projection -> fp8 down-projection with the sink -> combine."""
import numpy as np
import pytest
import torch

import oracle as O
from ep_synth import CONFIGS, TINY, make_inputs
from grouped_gemm_scatter_amd import EP_ERR_UNSUPPORTED, EpError
from gpu_helpers import compare_step, layout_picks, make_ctx, to_dev

pytestmark = pytest.mark.gpu

SHAPES = {
    "two_ranks_ragged": TINY.replace(n_ranks=2, n_experts_global=8, n_experts_local=4,
                                     tokens_per_rank=300, top_k=2, k=256, n=512, dtype="fp8",
                                     seed=71),
    "hot_expert_bands": TINY.replace(n_ranks=2, n_experts_global=8, n_experts_local=4,
                                     tokens_per_rank=1600, top_k=2, k=128, n=256,
                                     routing="zipf", n_forced_empty=1, dtype="fp8", seed=72),
    "many_experts": TINY.replace(n_ranks=8, n_experts_global=64, n_experts_local=8,
                                 tokens_per_rank=128, top_k=6, k=384, n=512, my_rank=3,
                                 dtype="fp8", seed=73),
}


def _h_bound(x1, x1s, w1, w1s, off, R):
    """Oracle h (binary32) and a bound on |h_gpu - h|: each of g, u is a sum of
    n = 128 + 2 + hidden/128 rounded binary32 operations on both sides, so it
    is within 2 gamma_n * sum |x w| of the other side's; |silu'| <= 1.1."""
    hidden = x1.shape[1]
    gu = O.expert_rows_fp8(x1, x1s, w1, w1s, off, R).astype(np.float64)
    mag = O.expert_rows_fp8(x1 & 0x7F, x1s, w1 & 0x7F, w1s, off, R).astype(np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    n = 128 + 2 + hidden // 128
    gam = 2 * 1.01 * n * 2.0 ** -24
    dg, du = gam * mag[:, :I], gam * mag[:, I:]
    h = O.expert_swiglu_fp8(x1, x1s, w1, w1s, off, R)
    bound = 1.1 * dg * (np.abs(u) + du) + np.abs(g / (1 + np.exp(-g))) * du \
        + 2 ** -20 * np.abs(h) + 1e-30
    return h, bound


def _compare(h_codes, h_scale, h_ref, bound, what):
    ref_codes, ref_scale = O.quantize_rows_e4m3(h_ref)
    assert h_codes.shape == ref_codes.shape and h_scale.shape == ref_scale.shape
    M, I = h_ref.shape
    # scales: amax / 448 of values each within its bound
    bmax = bound.reshape(M, I // 128, 128).max(axis=-1)
    assert np.all(np.abs(h_scale.astype(np.float64) - ref_scale) <= bmax / 448 * 1.01 +
                  2.0 ** -22 * ref_scale), what
    s = np.repeat(h_scale.astype(np.float64), 128, axis=1)
    dec = O.e4m3fn_to_f64(h_codes) * s
    v = np.abs(h_ref.astype(np.float64)) / s
    step = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3),
                    2.0 ** -9)
    # half a step at the value's binade (or the next one up), plus the sum bound
    allowed = step * s * (1 + 1e-6) + bound
    err = np.abs(dec - h_ref.astype(np.float64))
    assert np.all(err <= allowed), (what, float((err / allowed).max()))
    assert (h_codes == ref_codes).mean() >= 0.99, what


def _run_gpu(cfg, inp, ctx):
    ids = to_dev(inp.topk_ids.astype(np.int32))
    offsets, src_info = ctx.group(ids)
    M = int(offsets[-1].item())
    x1, x1s = inp.up_rows(layout_picks(offsets, src_info, cfg.n_ranks, M))
    w1, w1s = inp.up_weights()
    h = torch.full((max(M, 1), cfg.k), 0x7F, dtype=torch.uint8, device="cuda")
    hs = torch.full((max(M, 1), cfg.k // 128), float("nan"), dtype=torch.float32, device="cuda")
    ctx.up_swiglu_fp8(to_dev(x1) if M else None, to_dev(x1s) if M else None, to_dev(w1),
                      to_dev(w1s), offsets, M, h if M else None, hs if M else None)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    return M, h[:M].cpu().numpy(), hs[:M].cpu().numpy(), w1, w1s


def _oracle(cfg, inp, w1, w1s):
    off, src = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    x1, x1s = inp.up_rows(O.row_picks(off, src, cfg.n_ranks))
    return _h_bound(x1, x1s, w1, w1s, off, cfg.n_ranks)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_fp8_swiglu_matches_oracle(name):
    cfg = SHAPES[name]
    print(f"[case] fp8 swiglu {name} {cfg}", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    M, h, hs, w1, w1s = _run_gpu(cfg, inp, ctx)
    assert M > 0
    _compare(h, hs, *_oracle(cfg, inp, w1, w1s), name)


def test_fp8_swiglu_full_size_skewed_shape():
    cfg = CONFIGS["skewed_fp8"]
    print("[case] fp8 swiglu full size skewed_fp8", flush=True)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    M, h, hs, w1, w1s = _run_gpu(cfg, inp, ctx)
    print(f"[case] fp8 swiglu full size: oracle on {M} rows", flush=True)
    _compare(h, hs, *_oracle(cfg, inp, w1, w1s), "skewed_fp8")


def test_fp8_swiglu_quantiser_is_bit_exact_when_h_is_exact():
    """X1 = 1 everywhere; every gate row sums to 40 (expert 0) or 56 (expert 1),
    so silu(g) = g in binary32 on both sides; up rows sum to small signed
    integers: h = g * u exactly, and codes and scales must match bit for bit."""
    H, I, El, R = 256, 256, 2, 1
    cfg = TINY.replace(n_ranks=R, n_experts_global=El, n_experts_local=El, tokens_per_rank=300,
                       top_k=1, k=I, n=H, dtype="fp8", seed=74)
    one, neg = O.f32_to_e4m3fn(np.float32(1.0)), O.f32_to_e4m3fn(np.float32(-1.0))
    w1 = np.zeros((El, 2 * I, H), dtype=np.uint8)
    for e, gsum in enumerate([40, 56]):
        w1[e, :I, :gsum] = one
        for i in range(I):
            u = (i * 7 + e) % 13 - 6
            w1[e, I + i, :abs(u)] = one if u > 0 else neg
    w1s = np.ones((El, 2 * I // 128, H // 128), dtype=np.float32)
    ids = np.zeros((R, cfg.tokens_per_rank, 1), dtype=np.int32)
    ids[0, 170:, 0] = 1                                   # 170 rows of expert 0, 130 of expert 1
    off, src = O.group_local_picks(ids, El, 0)
    M = int(off[-1])
    x1 = np.full((M, H), one, dtype=np.uint8)
    x1s = np.ones((M, H // 128), dtype=np.float32)
    ctx = make_ctx(cfg)
    offsets, _ = ctx.group(to_dev(ids))
    h = torch.empty((M, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((M, I // 128), dtype=torch.float32, device="cuda")
    ctx.up_swiglu_fp8(to_dev(x1), to_dev(x1s), to_dev(w1), to_dev(w1s), offsets, M, h, hs)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    hv = O.expert_swiglu_fp8(x1, x1s, w1, w1s, off, R)
    assert np.array_equal(hv, np.rint(hv)) and np.abs(hv).max() == 56 * 6
    rc, rs = O.quantize_rows_e4m3(hv)
    assert np.array_equal(h.cpu().numpy(), rc)
    assert np.array_equal(hs.cpu().numpy(), rs)


def test_fp8_swiglu_rejects_bf16_handles():
    cfg = TINY
    ctx = make_ctx(cfg)
    z = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    s = torch.zeros(1 << 12, dtype=torch.float32, device="cuda")
    off = torch.zeros(cfg.n_experts_local * cfg.n_ranks + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(EpError) as e:
        ctx.up_swiglu_fp8(None, None, z, s, off, 0, None, None)
    assert e.value.code == EP_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["two_ranks_ragged", "many_experts"])
def test_fp8_tokens_through_dispatch_up_projection_sink_and_combine(name):
    cfg = SHAPES[name]          # hidden a multiple of 512: scale rows of whole 16-byte pieces
    print(f"[case] fp8 token chain {name}", flush=True)
    inp = make_inputs(cfg)
    R, T, N, I = cfg.n_ranks, cfg.tokens_per_rank, cfg.n, cfg.k
    ctx = make_ctx(cfg)
    ids = to_dev(inp.topk_ids.astype(np.int32))
    tw = to_dev(inp.topk_w.astype(np.float32))
    tok, tok_s = inp.tokens()
    offsets, src_info = ctx.group(ids)
    M = int(offsets[-1].item())
    x1 = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    x1s = torch.empty((M, N // 128), dtype=torch.float32, device="cuda")
    ctx.dispatch(to_dev(tok), offsets, src_info, M, x1)
    ctx.dispatch(to_dev(tok_s), offsets, src_info, M, x1s)
    w1, w1s = inp.up_weights()
    h = torch.empty((M, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((M, I // 128), dtype=torch.float32, device="cuda")
    ctx.up_swiglu_fp8(x1, x1s, to_dev(w1), to_dev(w1s), offsets, M, h, hs)
    out = torch.full((R, T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx.step(h, to_dev(inp.w), offsets, src_info, M, ids, tw, out, x_scale=hs,
             w_scale=to_dev(inp.w_scale))
    torch.cuda.synchronize()
    assert ctx.query_error() == 0

    off_o, src_o = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    x1_o = O.dispatch_rows(tok, off_o, src_o, R)
    x1s_o = O.dispatch_rows(tok_s, off_o, src_o, R)
    hv_o, bound = _h_bound(x1_o, x1s_o, w1, w1s, off_o, R)
    _compare(h.cpu().numpy(), hs.cpu().numpy(), hv_o, bound, f"{name} H")
    h_o, hs_o = O.quantize_rows_e4m3(hv_o)
    ref = O.run_step(topk_ids=inp.topk_ids, topk_w=inp.topk_w, x=h_o, x_scale=hs_o, w=inp.w,
                     w_scale=inp.w_scale, dtype="fp8", n_ranks=R,
                     n_experts_per_device=cfg.n_experts_local, top_k=cfg.top_k,
                     msg_bytes=cfg.msg, max_tokens_per_rank=T, my_rank=cfg.my_rank,
                     epoch=ctx.epoch)
    compare_step(ctx, ref, cfg, out, cfg.msg)

"""The slice-major weight layout (EP_FLAG_W_SLICE_MAJOR, ep_pack_weights):
the re-layout kernel is an exact permutation of W's elements, and a handle
that reads the re-laid weights gives the same step as the oracle, on the
small cases of every bf16 tile shape and at the full decode size, and byte for
byte the same receive buffers, control words and outputs as the row-major
handle at the full prefill size."""
import numpy as np
import pytest
import torch

from ep_synth import CONFIGS, make_inputs
from grouped_gemm_scatter_amd import EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EpError

pytestmark = pytest.mark.gpu

from gpu_helpers import compare_step, device_inputs, make_ctx, oracle_step  # noqa: E402
from test_gpu_parity import CASES  # noqa: E402

BF16_CASES = ["multi_tile_256", "tile_128_ragged", "zipf_empty_experts", "single_rank",
              "no_local_rows", "many_experts_ragged", "decode_ragged",
              "decode_zipf_empty_experts", "decode_two_slices", "split_tail_mixed"]


def _slice_major_host(w_bits):
    """[E][N][K] -> [E][K/64][N][64], by reshaping on the host."""
    E, N, K = w_bits.shape
    return np.ascontiguousarray(w_bits.reshape(E, N, K // 64, 64).transpose(0, 2, 1, 3))


@pytest.mark.parametrize("shape", [(1, 128, 64), (3, 256, 192), (5, 384, 640)])
def test_pack_weights_is_the_relayout(shape):
    E, N, K = shape
    print(f"[case] pack {shape}", flush=True)
    cfg = CASES["tiny"].replace(n_experts_local=E, n_experts_global=E * CASES["tiny"].n_ranks,
                                n=N, k=K)
    ctx = make_ctx(cfg)
    rng = np.random.default_rng(41 + E)
    w = rng.integers(0, 1 << 16, size=(E, N, K), dtype=np.uint16)
    packed = ctx.pack_weights(torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    got = packed.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, _slice_major_host(w))


def test_pack_weights_rejects_overlap_and_fp8():
    ctx = make_ctx(CASES["tiny"])
    E, N, K = CASES["tiny"].n_experts_local, CASES["tiny"].n, CASES["tiny"].k
    buf = torch.zeros(2 * E * N * K, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(EpError) as e:
        ctx.pack_weights(buf, out=buf[64:])
    assert e.value.code == EP_ERR_INVALID_ARG
    with pytest.raises(EpError) as e:
        make_ctx(CASES["fp8_multi_tile"], w_slice_major=True)
    assert e.value.code == EP_ERR_UNSUPPORTED
    f8 = make_ctx(CASES["fp8_multi_tile"])
    with pytest.raises(EpError) as e:
        f8.pack_weights(torch.zeros(f8.n_experts_per_device * f8.hidden_n * f8.hidden_k,
                                    dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == EP_ERR_UNSUPPORTED


def _step(cfg, slice_major, fused=False, inp=None):
    inp = inp or make_inputs(cfg)
    ctx = make_ctx(cfg, w_slice_major=slice_major)
    d = device_inputs(inp, ctx)
    w = ctx.pack_weights(d["w"]) if slice_major else d["w"]
    del d["w"]
    out = torch.full((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    ctx.step(d["x"], w, d["offsets"], d["src_info"], d["m_total"], d["topk_ids"], d["topk_w"],
             out, fused=fused)
    torch.cuda.synchronize()
    assert ctx.query_error() == 0
    return ctx, inp, out


@pytest.mark.parametrize("name", BF16_CASES)
def test_slice_major_step_matches_oracle(name):
    cfg = CASES[name]
    print(f"[case] slice-major {name} {cfg}", flush=True)
    ctx, inp, out = _step(cfg, True)
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)


@pytest.mark.parametrize("name", ["decode_ragged", "split_tail_mixed"])
def test_slice_major_fused_step_matches_oracle(name):
    cfg = CASES[name]
    print(f"[case] slice-major fused {name}", flush=True)
    ctx, inp, out = _step(cfg, True, fused=True)
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)


def test_slice_major_full_size_decode_matches_oracle():
    cfg = CONFIGS["deepseek_decode"]
    print("[case] slice-major full size deepseek_decode", flush=True)
    ctx, inp, out = _step(cfg, True)
    print("[case] slice-major full size deepseek_decode: oracle", flush=True)
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)


@pytest.mark.parametrize("name", ["deepseek_prefill", "qwen3_moe"])
def test_slice_major_full_size_equals_row_major(name):
    cfg = CONFIGS[name]
    print(f"[case] slice-major vs row-major full size {name}", flush=True)
    inp = make_inputs(cfg)
    a, _, out_a = _step(cfg, False, inp=inp)
    b, _, out_b = _step(cfg, True, inp=inp)
    # both handles are at epoch 1 and own separate buffers: compare on the device
    state_a = list(a.recv) + [a.words, out_a.view(torch.int16)]
    state_b = list(b.recv) + [b.words, out_b.view(torch.int16)]
    for i, (p, q) in enumerate(zip(state_a, state_b)):
        assert torch.equal(p, q), f"state {i} differs"


def _random_bf16_cases():
    from test_gpu_random_shapes import random_cases
    return {c.name: c for c in random_cases(n=16, seed=3031) if c.dtype == "bf16"}


RANDOM_BF16 = _random_bf16_cases()


@pytest.mark.parametrize("name", sorted(RANDOM_BF16))
def test_slice_major_random_shapes_match_oracle(name):
    cfg = RANDOM_BF16[name]
    print(f"[case] slice-major random {cfg}", flush=True)
    ctx, inp, out = _step(cfg, True, fused=name.endswith(("1", "5", "9")))
    compare_step(ctx, oracle_step(inp, epoch=ctx.epoch), cfg, out, cfg.msg, ctx.epoch)

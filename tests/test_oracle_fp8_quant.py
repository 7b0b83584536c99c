"""Pins of the oracle's fp8 re-quantisation and of its SwiGLU on fp8 operands
(the fp8 up-projection, whose output is the fp8 X of the down-projection):
the e4m3fn encoder against every finite code, against torch's own cast on
random values and on every midpoint between adjacent codes, and against the
tie rule by itself; the per-row block quantiser's scale, extremes, zeros and
error bound; the fp8 SwiGLU against float64 sums within the binary32 bound."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3fn_to_f64(codes)
    ok = ~np.isnan(vals)
    return codes[ok], vals[ok]


def test_encoder_round_trips_every_finite_code():
    codes, vals = _finite_codes()
    assert np.array_equal(O.f32_to_e4m3fn(vals.astype(np.float32)), codes)


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 100_000),          # normals
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 50_000),  # around the subnormals
                        rng.standard_normal(50_000) * 30]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(O.f32_to_e4m3fn(x), _torch_e4m3(x))


def test_midpoints_round_to_the_even_code():
    codes, vals = _finite_codes()
    pos = np.sort(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2                  # exact in float64 and in float32
    assert np.all(mids.astype(np.float32).astype(np.float64) == mids)
    both = np.concatenate([mids, -mids]).astype(np.float32)
    got = O.f32_to_e4m3fn(both)
    # the even code of each adjacent pair: mantissa LSB 0
    assert np.all((got & 1) == 0)
    assert np.array_equal(got, _torch_e4m3(both))
    # just off a midpoint goes to the nearer code
    lo = np.nextafter(mids.astype(np.float32), np.float32(0))
    hi = np.nextafter(mids.astype(np.float32), np.float32(1e9))
    assert np.array_equal(O.e4m3fn_to_f64(O.f32_to_e4m3fn(lo)), pos[:-1])
    assert np.array_equal(O.e4m3fn_to_f64(O.f32_to_e4m3fn(hi)), pos[1:])


def test_saturation_zero_and_sign():
    got = O.f32_to_e4m3fn(np.array([448, 463.9, 464, 1e9, -1e9, 0.0, -0.0], dtype=np.float32))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80]


def test_quantiser_scale_extremes_and_error():
    rng = np.random.default_rng(5)
    h = (rng.standard_normal((9, 384)) * rng.uniform(0.01, 300, (9, 1))).astype(np.float32)
    h[4, 128:256] = 0.0                            # a block of zeros
    codes, scale = O.quantize_rows_e4m3(h)
    assert codes.shape == h.shape and scale.shape == (9, 3) and scale.dtype == np.float32
    hb = h.reshape(9, 3, 128)
    amax = np.abs(hb).max(axis=-1)
    want = (amax / np.float32(448)).astype(np.float32)
    want[amax == 0] = 1
    assert np.array_equal(scale, want)
    assert np.all(codes[4, 128:256] == 0) and scale[4, 1] == 1
    dec = O.e4m3fn_to_f64(codes).reshape(9, 3, 128)
    # the largest magnitude of each non-zero block becomes +-448
    for m in range(9):
        for b in range(3):
            if amax[m, b] > 0:
                k = np.argmax(np.abs(hb[m, b]))
                assert abs(dec[m, b, k]) == 448
    # error: half a step of e4m3fn at the value's binade, in units of the scale
    v = hb.astype(np.float64) / scale[..., None]
    step = np.where(np.abs(v) >= 2.0 ** -6,
                    2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(dec - v) <= step / 2 * (1 + 1e-6))


def test_quantiser_blocks_are_independent():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((4, 256)).astype(np.float32)
    c0, s0 = O.quantize_rows_e4m3(h)
    h2 = h.copy()
    h2[:, 128:] *= 1000
    c1, s1 = O.quantize_rows_e4m3(h2)
    assert np.array_equal(c0[:, :128], c1[:, :128]) and np.array_equal(s0[:, 0], s1[:, 0])
    assert not np.array_equal(s0[:, 1], s1[:, 1])


def _groups(sizes, R=1):
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
        off.extend([off[-1]] * (R - 1))
    return np.array(off, dtype=np.int64)


@pytest.mark.parametrize("seed", range(2))
def test_fp8_swiglu_within_bound_of_float64_sums(seed):
    """Gate and up sums as the fp8 GEMM's binary32 form (within gamma_n of the
    float64 block sums, n = 128 + 2 + K/128 roundings), SiLU and the product in
    binary32: the bound carried through silu(g) * u, plus 8 ulp."""
    rng = np.random.default_rng(60 + seed)
    H, I, El, R = 256, 128, 3, 2
    sizes = [6, 0, 9]
    off = _groups(sizes, R)
    M = sum(sizes)
    x1, sx = O.quantize_rows_e4m3(rng.standard_normal((M, H)).astype(np.float32))
    w = (rng.standard_normal((El, 2 * I, H)) / math.sqrt(H)).astype(np.float32)
    w1 = np.empty((El, 2 * I, H), dtype=np.uint8)
    sw = np.empty((El, 2 * I // 128, H // 128), dtype=np.float32)
    for e in range(El):
        wb = w[e].reshape(2 * I // 128, 128, H // 128, 128)
        amax = np.abs(wb).max(axis=(1, 3))
        sw[e] = (amax / np.float32(448)).astype(np.float32)
        w1[e] = O.f32_to_e4m3fn(wb / sw[e][:, None, :, None]).reshape(2 * I, H)
    h32 = O.expert_swiglu_fp8(x1, sx, w1, sw, off, R)
    assert h32.dtype == np.float32 and h32.shape == (M, I)
    gu = O.expert_rows_fp8_f64(x1, sx, w1, sw, off, R)
    g, u = gu[:, :I], gu[:, I:]
    h64 = g / (1.0 + np.exp(-g)) * u
    xd = np.abs(O.e4m3fn_to_f64(x1))
    mag = np.zeros_like(gu)
    for e, (lo, hi) in enumerate([(0, 6), (6, 6), (6, 15)]):
        if hi == lo:
            continue
        wd = np.abs(O.e4m3fn_to_f64(w1[e]))                            # [2I][H]
        swr = np.repeat(sw[e], 128, axis=0)                             # [2I][H/128]
        for b in range(H // 128):
            ks = slice(b * 128, (b + 1) * 128)
            mag[lo:hi] += (sx[lo:hi, b:b + 1] * swr[:, b][None, :]) * (xd[lo:hi, ks] @ wd[:, ks].T)
    eps = 2.0 ** -24
    n = 128 + 2 + H // 128
    gamma = n * eps / (1 - n * eps)
    dg, du = gamma * mag[:, :I], gamma * mag[:, I:]
    bound = 1.1 * dg * (np.abs(u) + du) + np.abs(g / (1 + np.exp(-g))) * du \
        + 8 * eps * np.abs(h64) + 1e-30
    assert np.all(np.abs(h32.astype(np.float64) - h64) <= bound)


def test_fp8_swiglu_gate_up_order_and_expert():
    """One-hot rows: h = silu(w_gate) * w_up of the row's own expert, up rows after gate rows."""
    H, I = 128, 128
    w1 = np.zeros((2, 2 * I, H), dtype=np.uint8)
    one = O.f32_to_e4m3fn(np.float32(1.0))
    two = O.f32_to_e4m3fn(np.float32(2.0))
    w1[0, :I, 5] = one          # expert 0: gate 1, up 2 at column 5
    w1[0, I:, 5] = two
    w1[1, :I, 5] = two          # expert 1: gate 2, up 1
    w1[1, I:, 5] = one
    sw = np.ones((2, 2, 1), dtype=np.float32)
    x1 = np.zeros((2, H), dtype=np.uint8)
    x1[:, 5] = one
    sx = np.ones((2, 1), dtype=np.float32)
    h = O.expert_swiglu_fp8(x1, sx, w1, sw, np.array([0, 1, 2]), 1)
    silu = lambda g: g / (1 + math.exp(-g))
    assert np.allclose(h[0], silu(1.0) * 2.0, rtol=1e-6)
    assert np.allclose(h[1], silu(2.0) * 1.0, rtol=1e-6)

"""Pins of the oracle's number formats against torch's own casts and hand cases."""
import numpy as np
import pytest
import torch

import oracle as O


def test_bf16_decode_exhaustive():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = O.bf16_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def _torch_bf16_bits(v32):
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_on_binary32():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(5000) * 1e30).astype(np.float32),
            (rng.standard_normal(5000) * 1e-39).astype(np.float32),   # binary32 subnormals
            (rng.standard_normal(5000) * 1e-44).astype(np.float32),
            np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                      3.39e38, 1.1754944e-38], dtype=np.float32)]
    # exact ties: halfway between every pair of adjacent finite bf16 codes
    codes = np.arange(0, 0x7F80, dtype=np.uint32)
    ties = ((codes << 16) | 0x8000).view(np.float32)
    vals.append(np.concatenate([ties, -ties]))
    # one binary32 ulp either side of each tie
    vals.append(((codes << 16) | 0x7FFF).view(np.float32))
    vals.append(((codes << 16) | 0x8001).view(np.float32))
    v = np.concatenate(vals)
    got = O.f64_to_bf16(v.astype(np.float64))
    ref = _torch_bf16_bits(v)
    assert np.array_equal(got, ref)


def test_bf16_round_nan():
    assert O.f64_to_bf16(np.array([np.nan]))[0] & 0x7FFF == 0x7FC0


def test_bf16_round_is_single_rounding_from_f64():
    # a = 1 + 2^-7 (odd last bit) and b = 1 (even): values just above the
    # halfway point must round up even when binary32 would see an exact tie.
    one = 1.0
    ulp = 2.0 ** -7
    above_tie = one + ulp / 2 + 2.0 ** -40       # rounds to binary32 tie 1+2^-8
    assert O.f64_to_bf16(np.array([above_tie]))[0] == 0x3F81
    below_tie = one + ulp / 2 - 2.0 ** -40
    assert O.f64_to_bf16(np.array([below_tie]))[0] == 0x3F80
    assert O.f64_to_bf16(np.array([one + ulp / 2]))[0] == 0x3F80      # tie -> even
    assert O.f64_to_bf16(np.array([one + 1.5 * ulp]))[0] == 0x3F82    # tie -> even
    # smallest bf16 subnormal is 2^-133; half of it ties to zero, a bit more rounds up
    assert O.f64_to_bf16(np.array([2.0 ** -134]))[0] == 0x0000
    assert O.f64_to_bf16(np.array([2.0 ** -134 * (1 + 2 ** -20)]))[0] == 0x0001
    # rounding past the largest finite bf16 gives infinity, just below does not
    big = float(O.bf16_to_f64(np.array([0x7F7F], dtype=np.uint16))[0])
    half_ulp = 2.0 ** (127 - 8)
    assert O.f64_to_bf16(np.array([big + half_ulp]))[0] == 0x7F80
    assert O.f64_to_bf16(np.array([big + half_ulp * 0.99]))[0] == 0x7F7F
    assert O.f64_to_bf16(np.array([-1e300]))[0] == 0xFF80


def test_e4m3fn_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = O.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))
    assert np.nanmax(got) == 448.0
    assert got[1] == 2.0 ** -9          # smallest subnormal


@pytest.mark.parametrize("n_vals", [1000])
def test_bf16_round_trip_is_identity(n_vals):
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 0x7F80, n_vals).astype(np.uint16)
    assert np.array_equal(O.f64_to_bf16(O.bf16_to_f64(codes)), codes)

"""Pins of the oracle's combine, the binary32 fused multiply-add chain in
ascending pick order (oracle/combine.c): against a brute force that rounds
each step exactly with rational arithmetic, closed forms, and the float64
sum within the textbook error bound of a binary32 recursive sum."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

F32_MAX = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127


def round_f32(q: Fraction) -> float:
    """q rounded to the nearest binary32, ties to even (subnormals included,
    overflow to infinity)."""
    if q == 0:
        return 0.0
    neg = q < 0
    q = -q if neg else q
    e = q.numerator.bit_length() - q.denominator.bit_length()     # 2^e <= q < 2^(e+2)
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)                                                 # subnormal spacing 2^-149
    ulp = Fraction(2) ** (e - 23)
    n = q / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if v > F32_MAX:
        return -np.inf if neg else np.inf
    return -float(v) if neg else float(v)


def fmaf_exact(a: float, b: float, c: float) -> float:
    """a*b + c rounded once to binary32 (a, b, c binary32 values).  An exact
    zero result takes the sign rule of IEEE 754 addition: -0 only when both
    a*b and c are zeros of negative sign."""
    exact = Fraction(a) * Fraction(b) + Fraction(c)
    if exact == 0:
        prod_neg = (np.signbit(a) != np.signbit(b)) if (a == 0 or b == 0) else (a * b < 0)
        if a * b == 0 and c == 0 and prod_neg and np.signbit(c):
            return -0.0
        return 0.0
    return round_f32(exact)


def test_round_f32_agrees_with_numpy_on_doubles():
    # numpy's float64 -> float32 cast rounds to nearest even: a second opinion
    # on round_f32 for values a double holds
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 39, 2000),
                           [1 + 2 ** -24, 1 + 3 * 2 ** -24, 2 ** -149, 3 * 2 ** -150, 1e39]])
    for v in vals:
        with np.errstate(over="ignore"):
            want = np.float64(np.float32(v))
        assert round_f32(Fraction(float(v))) == want, v


@pytest.mark.parametrize("seed", range(3))
def test_combine_matches_exact_fmaf_chain(seed):
    """Random routing, weights and slot rows: every output equals the exactly
    rounded fused multiply-add chain over the local picks in ascending k."""
    rng = np.random.default_rng(60 + seed)
    R, T, k, El, Eg, n = 2, 5, 4, 3, 6, 16
    my = int(rng.integers(0, 2))
    ids = np.stack([np.stack([rng.permutation(Eg)[:k] for _ in range(T)])
                    for _ in range(R)]).astype(np.int32)
    tw = rng.uniform(0, 1, (R, T, k)).astype(np.float32)
    msg = 2 * n
    bufs = []
    slot_vals = rng.standard_normal((R, T, k, n)) * 10.0 ** rng.integers(-3, 4, (R, T, k, 1))
    slot_bits = O.f64_to_bf16(slot_vals)
    for rk in range(R):
        bufs.append(np.ascontiguousarray(slot_bits[rk]).view(np.uint8).reshape(-1).copy())
    got = O.combine_tokens(ids, tw, bufs, n_experts_per_device=El, my_rank=my, top_k=k,
                           msg_bytes=msg, n=n, as_f32=True)
    lo = my * El
    for rk in range(R):
        for t in range(T):
            acc = [0.0] * n
            for kk in range(k):
                if lo <= ids[rk, t, kk] < lo + El:
                    sv = O.bf16_to_f64(slot_bits[rk, t, kk])
                    acc = [fmaf_exact(float(tw[rk, t, kk]), float(sv[j]), acc[j])
                           for j in range(n)]
            assert np.array_equal(got[rk, t].astype(np.float64), np.array(acc)), (rk, t)


def test_fused_and_unfused_differ_where_the_exact_chain_says():
    """A case where one rounding and two roundings disagree: the combine must
    give the fused result."""
    w = np.float32(1 + 2 ** -23)
    s = 1 + 2 ** -7                        # a bf16 value; w * s needs 31 bits
    c_prev = -1.0                          # from an earlier pick: w0 * s0 = -1
    fused = fmaf_exact(float(w), s, c_prev)
    unfused = float(np.float32(np.float32(w) * np.float32(s)) + np.float32(c_prev))
    assert fused != unfused
    ids = np.array([[[0, 1]]], dtype=np.int32)
    tw = np.array([[[1.0, w]]], dtype=np.float32)
    rows = O.f64_to_bf16(np.array([[c_prev], [s]]))
    buf = np.ascontiguousarray(rows).view(np.uint8).reshape(-1).copy()
    got = O.combine_tokens(ids, tw, [buf], n_experts_per_device=2, my_rank=0, top_k=2,
                           msg_bytes=2, n=1, as_f32=True)
    assert float(got[0, 0, 0]) == fused


def test_combine_float32_sum_within_recursive_sum_bound():
    """Against the float64 sum: |acc - sum| <= gamma_k * sum |w s| with
    gamma_k = k u / (1 - k u), u = 2^-24 (a recursive binary32 sum)."""
    rng = np.random.default_rng(9)
    R, T, k, n = 1, 40, 8, 64
    ids = np.tile(np.arange(k, dtype=np.int32), (R, T, 1))
    tw = rng.uniform(0, 1, (R, T, k)).astype(np.float32)
    slot_bits = O.f64_to_bf16(rng.standard_normal((R, T, k, n)))
    buf = np.ascontiguousarray(slot_bits[0]).view(np.uint8).reshape(-1).copy()
    got = O.combine_tokens(ids, tw, [buf], n_experts_per_device=k, my_rank=0, top_k=k,
                           msg_bytes=2 * n, n=n, as_f32=True)[0].astype(np.float64)
    prods = tw[0][..., None].astype(np.float64) * O.bf16_to_f64(slot_bits[0])
    exact = prods.sum(axis=1)
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    assert np.all(np.abs(got - exact) <= gamma * np.abs(prods).sum(axis=1))


def test_token_without_local_picks_is_positive_zero():
    ids = np.array([[[5, 6], [0, 7]]], dtype=np.int32)
    tw = np.array([[[0.5, 0.5], [1.0, 0.0]]], dtype=np.float32)
    row = O.f64_to_bf16(np.array([[-0.0, -1.0], [2.0, 3.0]]))   # slots of token 0 never read
    buf = np.concatenate([np.ascontiguousarray(row).view(np.uint8).reshape(-1),
                          np.ascontiguousarray(O.f64_to_bf16(np.array([[-0.0, 4.0], [9.0, 9.0]])))
                          .view(np.uint8).reshape(-1)])
    out = O.combine_tokens(ids, tw, [buf], n_experts_per_device=2, my_rank=0, top_k=2,
                           msg_bytes=4, n=2)
    assert out[0, 0].tolist() == [0, 0]                 # +0, sign bit clear
    # token 1: pick 0 is local with weight 1: fmaf(1, -0, +0) = +0 and 4 exactly
    assert out[0, 1].tolist() == [0, int(O.f64_to_bf16(np.array([4.0]))[0])]

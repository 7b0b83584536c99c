"""Pins of the oracle's expert GEMM (bf16 and blockwise fp8), in both its
forms: the binary32-accumulating one the parity tests compare with, and the
float64 reference.  Closed forms (identity, one-hot rows) and power-of-two
scaling are exact in both; the float64 form matches pure-Python brute force
on tiny shapes; the binary32 form stays within the textbook bound of a
binary32 inner product of length K, gamma_K * sum |x w|, of the brute force."""
import numpy as np
import pytest
import torch

import oracle as O


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _groups(sizes, R=1):
    """offsets for groups of the given sizes, all rows on rank 0 of R ranks."""
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
        off.extend([off[-1]] * (R - 1))
    return np.array(off, dtype=np.int64)


GEMMS = {"f32": O.expert_rows_bf16, "f64": O.expert_rows_bf16_f64}


def _round(y):
    return O.f64_to_bf16(np.asarray(y, dtype=np.float64))


@pytest.mark.parametrize("form", sorted(GEMMS))
def test_identity_weight_is_exact(form):
    rng = np.random.default_rng(3)
    K = N = 96
    x = _bf16(rng.standard_normal((40, K)))
    w = _bf16(np.stack([np.eye(N, K), np.eye(N, K)]))
    off = _groups([25, 15], R=2)
    y = GEMMS[form](x, w, off, 2)
    assert np.array_equal(_round(y), x)


@pytest.mark.parametrize("form", sorted(GEMMS))
def test_one_hot_rows_pick_weight_columns(form):
    rng = np.random.default_rng(4)
    K, N, El = 64, 48, 3
    w = _bf16(rng.standard_normal((El, N, K)))
    sizes = [K, 0, K]
    off = _groups(sizes)
    M = sum(sizes)
    x = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        x[m, m % K] = 1.0
    y = GEMMS[form](_bf16(x), w, off, 1)
    for m in range(M):
        e = 0 if m < K else 2
        # row m selects row (m % K) of the logical K x N matrix W_e,
        # i.e. column (m % K) of its [N][K] storage
        assert np.array_equal(_round(y[m]), w[e][:, m % K])


@pytest.mark.parametrize("form", sorted(GEMMS))
def test_power_of_two_scaling_is_exact(form):
    rng = np.random.default_rng(5)
    K, N = 80, 40
    x = _bf16(rng.standard_normal((30, K)))
    w = rng.standard_normal((2, N, K)).astype(np.float32)
    off = _groups([10, 20])
    y1 = GEMMS[form](x, _bf16(w), off, 1)
    y8 = GEMMS[form](x, _bf16(w * 8), off, 1)
    assert np.array_equal(y8, 8 * y1)


def _brute_bf16(x, w, off, R, rows):
    out = []
    El = w.shape[0]
    for m in rows:
        e = next(e for e in range(El) if off[e * R] <= m < off[(e + 1) * R])
        xr = [float(v) for v in O.bf16_to_f64(x[m])]
        we = O.bf16_to_f64(w[e])
        out.append([sum(xr[k] * float(we[n][k]) for k in range(len(xr))) for n in range(w.shape[1])])
    return np.array(out)


@pytest.mark.parametrize("seed", range(4))
def test_bf16_gemm_matches_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    R, El = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    K, N = int(rng.integers(1, 40)), int(rng.integers(1, 24))
    sizes = rng.integers(0, 6, El * R)
    off = np.concatenate([[0], np.cumsum(sizes)])
    M = int(off[-1])
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((El, N, K)))
    rows = rng.permutation(M)[: min(M, 9)]
    y = O.expert_rows_bf16_f64(x, w, off, R, rows)
    b = _brute_bf16(x, w, off, R, rows)
    bound = 1e-13 * (np.abs(O.bf16_to_f64(x[rows])).sum(1, keepdims=True) + 1) * 8
    assert np.all(np.abs(y - b) <= bound)


def _abs_products(x, w, off, R, rows):
    """sum_k |x[m][k] w_e[k][n]| per requested row, for the error bounds."""
    El = w.shape[0]
    out = []
    for m in rows:
        e = next(e for e in range(El) if off[e * R] <= m < off[(e + 1) * R])
        out.append(np.abs(O.bf16_to_f64(w[e])) @ np.abs(O.bf16_to_f64(x[m])))
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_bf16_gemm_f32_within_inner_product_bound(seed):
    """Every binary32 result lies within gamma_K * sum_k |x w| of the brute-force
    exact sum (products of bf16 values are exact in binary32, so only the K
    additions round), on ragged groups over several ranks, K up to 300."""
    rng = np.random.default_rng(90 + seed)
    R, El = int(rng.integers(1, 4)), int(rng.integers(2, 5))
    K, N = int(rng.integers(1, 300)), int(rng.integers(1, 40))
    sizes = rng.integers(0, 7, El * R)
    off = np.concatenate([[0], np.cumsum(sizes)])
    M = int(off[-1])
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((El, N, K)))
    rows = rng.permutation(M)[: min(M, 12)]
    y = O.expert_rows_bf16(x, w, off, R, rows).astype(np.float64)
    assert O.expert_rows_bf16(x, w, off, R, rows).dtype == np.float32
    b = _brute_bf16(x, w, off, R, rows)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    s = _abs_products(x, w, off, R, rows)
    assert np.all(np.abs(y - b) <= gamma * s + 1e-300)


def _e4m3(a):
    a = np.clip(a, -448, 448).astype(np.float32)
    return torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _brute_fp8(xq, sx, wq, sw, e, m, n):
    acc = 0.0
    K = xq.shape[1]
    for b in range(K // 128):
        part = 0.0
        for k in range(b * 128, (b + 1) * 128):
            part += float(O.e4m3fn_to_f64(xq[m, k])) * float(O.e4m3fn_to_f64(wq[e, n, k]))
        acc += float(sx[m, b]) * float(sw[e, n // 128, b]) * part
    return acc


def test_fp8_blockwise_matches_brute_force():
    rng = np.random.default_rng(20)
    K, N, El = 256, 128, 2
    sizes = [3, 2]
    off = _groups(sizes)
    M = sum(sizes)
    xq = _e4m3(rng.standard_normal((M, K)) * 30)
    wq = _e4m3(rng.standard_normal((El, N, K)) * 30)
    sx = rng.uniform(0.01, 2, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.01, 2, (El, N // 128, K // 128)).astype(np.float32)
    y = O.expert_rows_fp8_f64(xq, sx, wq, sw, off, 1)
    y32 = O.expert_rows_fp8(xq, sx, wq, sw, off, 1).astype(np.float64)
    xd = O.e4m3fn_to_f64(xq)
    u = 2.0 ** -24
    for m in range(M):
        e = 0 if m < 3 else 1
        for n in rng.permutation(N)[:6]:
            ref = _brute_fp8(xq, sx, wq, sw, e, m, n)
            assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref)) * 1e3
            # binary32 form: each block's 128 exact products summed (128 roundings),
            # scaled (2 roundings) and added (K/128 roundings)
            mag = sum(float(sx[m, b]) * float(sw[e, n // 128, b]) *
                      float(np.abs(xd[m, b * 128:(b + 1) * 128]) @
                            np.abs(O.e4m3fn_to_f64(wq[e, n, b * 128:(b + 1) * 128])))
                      for b in range(K // 128))
            g = 140 * u / (1 - 140 * u)
            assert abs(y32[m, n] - ref) <= g * mag


def test_fp8_block_scale_acts_on_its_block_only():
    rng = np.random.default_rng(21)
    K, N = 384, 256
    off = _groups([4])
    xq = _e4m3(rng.standard_normal((4, K)) * 20)
    wq = _e4m3(rng.standard_normal((1, N, K)) * 20)
    sx = np.ones((4, 3), np.float32)
    sw = np.ones((1, 2, 3), np.float32)
    base = O.expert_rows_fp8_f64(xq, sx, wq, sw, off, 1)
    # unit scales: the plain product of decoded codes; the binary32 form gives
    # the same as the plain binary32 product of the decoded codes
    xd, wd = O.e4m3fn_to_f64(xq), O.e4m3fn_to_f64(wq[0])
    b32 = O.expert_rows_fp8(xq, sx, wq, sw, off, 1)
    p32 = np.zeros_like(b32)
    for b in range(3):
        p32 += xd[:, b * 128:(b + 1) * 128].astype(np.float32) @ \
            wd[:, b * 128:(b + 1) * 128].astype(np.float32).T
    assert np.array_equal(b32, p32)
    assert np.array_equal(base, xd @ wd.T) or np.allclose(base, xd @ wd.T, rtol=0, atol=1e-9)
    # doubling activation scale of block 1 adds exactly block 1's contribution
    sx2 = sx.copy()
    sx2[:, 1] = 2
    y2 = O.expert_rows_fp8_f64(xq, sx2, wq, sw, off, 1)
    blk1 = xd[:, 128:256] @ wd[:, 128:256].T
    assert np.allclose(y2 - base, blk1, rtol=0, atol=1e-9)
    # weight scale of n-block 0, k-block 2 only touches columns 0..127
    sw2 = sw.copy()
    sw2[0, 0, 2] = 4
    y3 = O.expert_rows_fp8_f64(xq, sx, wq, sw2, off, 1)
    blk2 = xd[:, 256:] @ wd[:, 256:].T
    assert np.allclose((y3 - base)[:, :128], 3 * blk2[:, :128], rtol=0, atol=1e-9)
    assert np.array_equal(y3[:, 128:], base[:, 128:])
    # binary32 form: the same block scale leaves the other n-block bit-identical
    y3_32 = O.expert_rows_fp8(xq, sx, wq, sw2, off, 1)
    assert np.array_equal(y3_32[:, 128:], b32[:, 128:])
    assert not np.array_equal(y3_32[:, :128], b32[:, :128])

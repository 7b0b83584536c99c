"""Pins of the oracle's up-projection with SwiGLU (the expert FFN's first GEMM):
torch's own SiLU on separately computed gate and up products, one-hot rows that
select weight columns, the zeros and asymptotes of SiLU, and the gate/up order."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _groups(sizes, R=1):
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
        off.extend([off[-1]] * (R - 1))
    return np.array(off, dtype=np.int64)


@pytest.mark.parametrize("seed", range(3))
def test_matches_torch_silu_on_gate_and_up(seed):
    rng = np.random.default_rng(40 + seed)
    H, I, El, R = 96, 32, 3, 2
    sizes = [7, 0, 12]
    off = _groups(sizes, R)
    M = sum(sizes)
    x1 = _bf16(rng.standard_normal((M, H)))
    w1 = _bf16(rng.standard_normal((El, 2 * I, H)) / math.sqrt(H))
    h = O.expert_swiglu_f64(x1, w1, off, R)
    xt = torch.from_numpy(O.bf16_to_f64(x1))
    for e, (lo, hi) in enumerate([(0, 7), (7, 7), (7, 19)]):
        if lo == hi:
            continue
        wt = torch.from_numpy(O.bf16_to_f64(w1[e]))           # [2I][H]
        gate = xt[lo:hi] @ wt[:I].T
        up = xt[lo:hi] @ wt[I:].T
        ref = (torch.nn.functional.silu(gate) * up).numpy()
        np.testing.assert_allclose(h[lo:hi], ref, rtol=1e-12, atol=1e-12)


def test_one_hot_rows_select_gate_and_up_columns():
    rng = np.random.default_rng(7)
    H, I = 40, 16
    w1 = _bf16(rng.standard_normal((2, 2 * I, H)))
    off = _groups([H, H])
    x = np.zeros((2 * H, H), dtype=np.float32)
    for m in range(2 * H):
        x[m, m % H] = 1.0
    h = O.expert_swiglu_f64(_bf16(x), w1, off, 1)
    for m in range(2 * H):
        e, k = m // H, m % H
        g = torch.from_numpy(O.bf16_to_f64(w1[e][:I, k]))
        u = torch.from_numpy(O.bf16_to_f64(w1[e][I:, k]))
        np.testing.assert_allclose(h[m], (torch.nn.functional.silu(g) * u).numpy(), rtol=1e-14)


def test_zero_gate_or_zero_up_gives_exact_zero():
    rng = np.random.default_rng(8)
    H, I = 32, 8
    x1 = _bf16(rng.standard_normal((6, H)))
    w = rng.standard_normal((1, 2 * I, H)).astype(np.float32)
    wg0 = w.copy(); wg0[0, :I] = 0
    wu0 = w.copy(); wu0[0, I:] = 0
    off = _groups([6])
    assert np.all(O.expert_swiglu_f64(x1, _bf16(wg0), off, 1) == 0)
    assert np.all(O.expert_swiglu_f64(x1, _bf16(wu0), off, 1) == 0)


def test_silu_asymptotes_and_gate_up_order():
    # one row, one input: g = a * wg, u = a * wu with exact bf16 products
    x1 = _bf16(np.array([[1.0]]))
    off = _groups([1])
    for g, u in [(30.0, 0.5), (-30.0, 3.0), (0.5, 2.0)]:
        w1 = _bf16(np.array([[[g], [u]]]))
        h = float(O.expert_swiglu_f64(x1, w1, off, 1)[0, 0])
        if g > 20:
            assert abs(h - g * u) <= 1e-11 * abs(g * u)      # silu(g) -> g
        elif g < -20:
            assert abs(h) <= 1e-11                            # silu(g) -> 0
        else:
            assert h == pytest.approx(float(torch.nn.functional.silu(torch.tensor(g, dtype=torch.float64))) * u, rel=1e-14)
        # exchanging the gate and up rows changes the result
        swapped = float(O.expert_swiglu_f64(x1, _bf16(np.array([[[u], [g]]])), off, 1)[0, 0])
        assert swapped != pytest.approx(h, rel=1e-3)


@pytest.mark.parametrize("seed", range(3))
def test_f32_form_within_bound_of_the_f64_form(seed):
    """The binary32 form (the one parity compares with): gate and up each within
    gamma_H * sum |x w| of the float64 sums, then SiLU and the product in
    binary32, a few rounding errors more: the result stays within that bound
    carried through silu(g) * u, plus 8 ulp of the result."""
    rng = np.random.default_rng(50 + seed)
    H, I, El, R = 160, 24, 3, 2
    sizes = [9, 0, 14]
    off = _groups(sizes, R)
    M = sum(sizes)
    x1 = _bf16(rng.standard_normal((M, H)))
    w1 = _bf16(rng.standard_normal((El, 2 * I, H)) / math.sqrt(H))
    h32 = O.expert_swiglu(x1, w1, off, R)
    assert h32.dtype == np.float32
    h64 = O.expert_swiglu_f64(x1, w1, off, R)
    gu = O.expert_rows_bf16_f64(x1, w1, off, R)
    g, u = gu[:, :I], gu[:, I:]
    xa = np.abs(O.bf16_to_f64(x1))
    absw = np.zeros_like(gu)
    for e, (lo, hi) in enumerate([(0, 9), (9, 9), (9, 23)]):
        if hi > lo:
            absw[lo:hi] = xa[lo:hi] @ np.abs(O.bf16_to_f64(w1[e])).T
    eps = 2.0 ** -24
    gamma = H * eps / (1 - H * eps)
    dg, du = gamma * absw[:, :I], gamma * absw[:, I:]
    # |d silu/dg| <= 1.1 everywhere
    bound = 1.1 * dg * (np.abs(u) + du) + np.abs(g * (1 / (1 + np.exp(-g)))) * du \
        + 8 * eps * np.abs(h64) + 1e-30
    assert np.all(np.abs(h32.astype(np.float64) - h64) <= bound)


def test_f32_form_one_hot_rows_are_single_products():
    """One-hot X1 rows make gate and up single exact products; the binary32
    SiLU product then agrees with torch's float32 SiLU to within 4 ulp."""
    rng = np.random.default_rng(57)
    H, I = 40, 16
    w1 = _bf16(rng.standard_normal((1, 2 * I, H)))
    off = _groups([H])
    x = np.eye(H, dtype=np.float32)
    h = O.expert_swiglu(_bf16(x), w1, off, 1)
    for m in range(H):
        g = torch.from_numpy(O.bf16_to_f64(w1[0][:I, m]).astype(np.float32))
        u = torch.from_numpy(O.bf16_to_f64(w1[0][I:, m]).astype(np.float32))
        ref = (torch.nn.functional.silu(g) * u).numpy()
        np.testing.assert_allclose(h[m], ref, rtol=4 * 2.0 ** -23, atol=1e-37)

"""The seeded generator: deterministic, X rows keyed by pick (independent of
which picks are asked for and in which order), routing of the stated shape,
and the skewed workload ragged with empty experts."""
import numpy as np
import pytest

import oracle as O
from ep_synth import CONFIGS, SKEWED_FP8, TINY, make_inputs, make_routing


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_routing_shape_and_weights(name):
    cfg = CONFIGS[name]
    ids, tw = make_routing(cfg)
    R, T, k = cfg.n_ranks, cfg.tokens_per_rank, cfg.top_k
    assert ids.shape == (R, T, k) and tw.shape == (R, T, k)
    assert ids.dtype == np.int32 and tw.dtype == np.float32
    assert ids.min() >= 0 and ids.max() < cfg.n_experts_global
    for row in ids.reshape(-1, k)[:: max(1, R * T // 500)]:
        assert len(set(row.tolist())) == k                 # distinct picks
    assert np.allclose(tw.sum(-1), 1.0, atol=1e-6)


def test_generator_is_deterministic():
    a, b = make_inputs(TINY), make_inputs(TINY)
    for f in ("topk_ids", "topk_w", "w"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    picks = [[0, 0, 0], [1, 7, 1]]
    assert np.array_equal(a.rows(picks)[0], b.rows(picks)[0])
    c = make_inputs(TINY.replace(seed=1))
    assert not np.array_equal(a.rows(picks)[0], c.rows(picks)[0])
    assert not np.array_equal(a.topk_ids, c.topk_ids)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rows_are_keyed_by_pick(dtype):
    cfg = TINY.replace(k=256, dtype=dtype, seed=4)
    inp = make_inputs(cfg)
    picks = np.array([[r, t, k] for r in range(2) for t in range(8) for k in range(2)])
    x, xs = inp.rows(picks)
    order = np.random.default_rng(0).permutation(len(picks))[:11]
    x2, xs2 = inp.rows(picks[order])
    assert np.array_equal(x2, x[order])
    if dtype == "fp8":
        assert np.array_equal(xs2, xs[order])
    # distinct picks get distinct rows
    assert len({bytes(r) for r in x}) == len(picks)
    up = inp.up_rows(picks[:3])
    if dtype == "fp8":
        (up, ups), (one, ones) = up, inp.up_rows(picks[2:3])
        assert ups.shape == (3, cfg.n // 128) and np.array_equal(ones[0], ups[2])
    else:
        one = inp.up_rows(picks[2:3])
    assert up.shape == (3, cfg.n) and np.array_equal(one[0], up[2])


def test_skewed_routing_is_ragged_with_empty_experts():
    ids, _ = make_routing(SKEWED_FP8)
    off, _ = O.group_local_picks(ids, SKEWED_FP8.n_experts_local, SKEWED_FP8.my_rank)
    sizes = np.diff(off[:: SKEWED_FP8.n_ranks])
    assert (sizes == 0).sum() == SKEWED_FP8.n_forced_empty
    assert sizes.max() > 8 * np.median(sizes[sizes > 0])
    assert np.any(sizes % 256 != 0)


def test_fp8_quantisation_bounds():
    cfg = TINY.replace(dtype="fp8", k=256, n=256, seed=2)
    inp = make_inputs(cfg)
    x, xs = inp.rows([[r, t, k] for r in range(2) for t in range(8) for k in range(2)])
    xd = O.e4m3fn_to_f64(x).reshape(x.shape[0], 2, 128)
    assert np.all(np.abs(xd) <= 448)
    # the block maximum is encoded as +-448 (amax / scale = 448 exactly or nearly)
    assert np.all(np.abs(xd).max(-1) >= 416)
    assert xs.shape == (x.shape[0], 2) and inp.w_scale.shape == (2, 2, 2)

"""Seeded random shapes through the whole step on the GPU, compared with the
oracle like the named parity cases (placement, counts, flags and counters
exact; values within tolerance), plus the GPU grouping of the same routing.
The shapes vary the rank count, local experts, tokens, top_k, K, N, dtype,
routing (zipf with forced-empty experts) and this GPU's rank."""
import numpy as np
import pytest

from ep_synth import TINY


def random_cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        R = int(rng.integers(1, 9))
        El = int(rng.integers(1, 9))
        Eg = R * El
        fp8 = bool(rng.random() < 0.3)
        zipf = bool(rng.random() < 0.3)
        empty = int(rng.integers(0, El)) if zipf else 0
        k = int(rng.integers(1, min(8, Eg - empty) + 1))
        K = int(128 * rng.integers(1, 5)) if fp8 else int(64 * rng.integers(1, 9))
        cases.append(TINY.replace(
            name=f"random_{i}", n_ranks=R, n_experts_global=Eg, n_experts_local=El,
            tokens_per_rank=int(rng.integers(1, 400)), top_k=k, k=K,
            n=int(128 * rng.integers(1, 7)), dtype="fp8" if fp8 else "bf16",
            routing="zipf" if zipf else "uniform", n_forced_empty=empty,
            my_rank=int(rng.integers(0, R)), seed=100 + i))
    return cases


CASES = {c.name: c for c in random_cases()}


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(CASES))
def test_random_shape_step_and_grouping(name):
    import torch

    import oracle as O
    from ep_synth import make_inputs
    from gpu_helpers import make_ctx
    from test_gpu_parity import _run

    cfg = CASES[name]
    print(f"[case] {cfg}", flush=True)
    _run(cfg)
    inp = make_inputs(cfg)
    ctx = make_ctx(cfg)
    off, src = ctx.group(torch.from_numpy(inp.topk_ids.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    want_off, want_src = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
    assert np.array_equal(off.cpu().numpy(), want_off)
    m = int(want_off[-1])
    assert np.array_equal(src[:m].cpu().numpy(), want_src)


def test_random_shapes_are_valid_inputs():
    """CPU: every random shape draws, and the oracle runs its whole step on it
    (so the GPU cases exercise what they claim: several shapes hold rows)."""
    import oracle as O
    from ep_synth import make_inputs
    with_rows = 0
    for cfg in CASES.values():
        inp = make_inputs(cfg)
        off, _ = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
        with_rows += int(off[-1]) > 0
    assert with_rows >= len(CASES) - 2

"""Seeded random shapes large enough for the 256-column tile (hundreds to a few
thousand rows per expert, ragged tails, partial last rounds), each run through a
random mode of the step: rank-level or per-expert completion, agent or system
scope, two launches or the fused launch, the default kernels or the send-wave
kernel (bf16), padded or unpadded slots, one to three consecutive epochs.
Compared with the oracle like the named parity cases: placement, counts,
flags and counters exact, values within tolerance."""
import numpy as np
import pytest

from ep_synth import TINY


def random_mode_cases(n=10, seed=7):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        R = int(rng.integers(2, 9))
        El = int(rng.integers(1, 5))
        Eg = R * El
        fp8 = bool(rng.random() < 0.3)
        zipf = bool(rng.random() < 0.4)
        empty = int(rng.integers(0, El)) if zipf and El > 1 else 0
        k = int(rng.integers(1, min(8, Eg - empty) + 1))
        K = int(128 * rng.integers(1, 4)) if fp8 else int(64 * rng.integers(1, 7))
        N = int(256 * rng.integers(1, 5))
        T = int(rng.integers(300, 2000))
        cfg = TINY.replace(
            name=f"random_mode_{i}", n_ranks=R, n_experts_global=Eg, n_experts_local=El,
            tokens_per_rank=T, top_k=k, k=K, n=N, dtype="fp8" if fp8 else "bf16",
            routing="zipf" if zipf else "uniform", n_forced_empty=empty,
            my_rank=int(rng.integers(0, R)), seed=300 + i)
        mode = {
            "per_expert_release": bool(rng.random() < 0.3),
            "system_scope": bool(rng.random() < 0.3),
            "fused": bool(rng.random() < 0.3),
            "epochs": int(rng.integers(1, 4)),
            "pad": int(16 * rng.integers(0, 3)),
        }
        mode["send_waves"] = 4 if (not fp8 and not mode["fused"] and rng.random() < 0.4) else 0
        cases.append((cfg, mode))
    return cases


CASES = {c.name: (c, m) for c, m in random_mode_cases()}


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(CASES))
def test_random_shape_in_a_random_mode(name):
    from test_gpu_parity import _run

    cfg, mode = CASES[name]
    print(f"[case] {cfg} {mode}", flush=True)
    kw = {k: v for k, v in mode.items() if k in ("per_expert_release", "system_scope")}
    if mode["send_waves"]:
        kw["send_waves"] = mode["send_waves"]
    _run(cfg, msg_bytes=2 * cfg.n + mode["pad"], epochs=mode["epochs"], fused=mode["fused"], **kw)


def test_random_modes_cover_the_tiles_and_modes():
    """CPU: the random cases hold rows, reach the 256-column tile's sizes and
    cover every mode at least once."""
    import oracle as O
    from ep_synth import make_inputs
    big, modes = 0, set()
    for cfg, mode in CASES.values():
        inp = make_inputs(cfg)
        off, _ = O.group_local_picks(inp.topk_ids, cfg.n_experts_local, cfg.my_rank)
        rows = np.diff(off[::cfg.n_ranks])
        big += int(rows.max(initial=0) > 256)
        modes |= {k for k, v in mode.items() if v and k in ("per_expert_release", "system_scope",
                                                           "fused", "send_waves", "pad")}
        modes |= {"fp8"} if cfg.dtype == "fp8" else set()
        modes |= {"epochs"} if mode["epochs"] > 1 else set()
    assert big >= 5
    assert modes == {"per_expert_release", "system_scope", "fused", "send_waves", "pad", "fp8",
                     "epochs"}, modes

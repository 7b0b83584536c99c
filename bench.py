"""Benchmark of one EP-combine step on one MI355X.

A step is one pass of the whole path on one batch of synthetic input: the
grouped GEMM with the in-epilogue row scatter and fused completion signals
(ep_grouped_gemm_scatter) followed by the consumer combine (ep_combine_reduce),
both through the C ABI, inputs resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "grouped_gemm_scatter_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# sources of each GEMM kernel: measured traffic is only reported while they are unchanged
KERNEL_SOURCES = {
    "bf16": ["gemm_scatter.hip", "gemm_common.h", "ep_device.h", "ep_kernels.h"],
    "fp8": ["gemm_scatter_fp8.hip", "gemm_common.h", "ep_device.h", "ep_kernels.h"],
}
COPY_PROBE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup: the GPU takes tens of "
                         "milliseconds of sustained load to reach its steady clocks")
    ap.add_argument("--config", default="deepseek_prefill")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens per rank in the oracle's timed sample (0: all of them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--steps-only", action="store_true",
                    help="time the EP-combine steps alone: no local-C, epilogue-only or "
                         "per-expert launches (used for the hardware-counter runs, so that "
                         "every launch of the GEMM kernel is a step's)")
    ap.add_argument("--no-up-proj", action="store_true",
                    help="skip the up-projection + SwiGLU GEMM measurement")
    ap.add_argument("--no-per-expert", action="store_true",
                    help="skip timing the per-expert completion variant beside the main step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the HBM byte counters)")
    return ap.parse_args()


def kernel_digest(dtype):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[dtype]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(cfg):
    """HBM bytes per GEMM launch from the committed counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel factor),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(PROFILES, f"traffic_{cfg.name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != kernel_digest(cfg.dtype):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = COPY_PROBE_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES,
                      "copy_probe_bytes_written": COPY_PROBE_BYTES, "launches": 5}))


def step_bytes(cfg, M, n_nonempty):
    elt = 1 if cfg.dtype == "fp8" else 2
    K, N, R, T, k = cfg.k, cfg.n, cfg.n_ranks, cfg.tokens_per_rank, cfg.top_k
    scales = 0
    if cfg.dtype == "fp8":
        scales = M * (K // 128) * 4 + n_nonempty * (N // 128) * (K // 128) * 4
    gemm = n_nonempty * K * N * elt + M * K * elt + M * 2 * N + scales
    scatter = M * 2 * N
    combine = M * 2 * N + R * T * 2 * N + R * T * k * 8
    return gemm, scatter, combine


def cpu_baseline(inp, tokens):
    """Times the oracle on a token-prefix sample of the same workload."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cfg = inp.cfg
    S = cfg.tokens_per_rank if tokens <= 0 else min(tokens, cfg.tokens_per_rank)
    keep = inp.src_info[:, 0] < S
    x = inp.x[keep]
    t0 = time.perf_counter()
    res = O.run_step(topk_ids=inp.topk_ids[:, :S], topk_w=inp.topk_w[:, :S], x=x, w=inp.w,
                     n_ranks=cfg.n_ranks, n_experts_per_device=cfg.n_experts_local,
                     top_k=cfg.top_k, msg_bytes=cfg.msg, max_tokens_per_rank=S,
                     my_rank=cfg.my_rank, dtype=cfg.dtype,
                     x_scale=None if inp.x_scale is None else inp.x_scale[keep],
                     w_scale=inp.w_scale)
    dt = time.perf_counter() - t0
    Ms = int(res["offsets"][-1])
    flops = 2.0 * Ms * cfg.k * cfg.n
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"all {S} tokens per rank" if S == cfg.tokens_per_rank else
                       f"first {S} of {cfg.tokens_per_rank} tokens per rank") +
                      f": {Ms} rows, full grouping+GEMM+scatter+counts+combine, {dt:.2f} s"}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the EP combine; runs on more than one "
              "GPU are not part of this build (each GPU would run the same step on its own "
              "expert slice).", file=sys.stderr)
        sys.exit(2)

    import torch

    from ep_synth import config_by_name, make_inputs
    from grouped_gemm_scatter_amd import EpCombine

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = config_by_name(args.config)
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg)
    M = inp.m_total
    fp8 = cfg.dtype == "fp8"
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp.x).view(torch.uint8 if fp8 else torch.bfloat16).to(dev)
    w = torch.from_numpy(inp.w).view(torch.uint8 if fp8 else torch.bfloat16).to(dev)
    xs = torch.from_numpy(inp.x_scale).to(dev) if fp8 else None
    ws = torch.from_numpy(inp.w_scale).to(dev) if fp8 else None
    offsets = torch.from_numpy(inp.offsets.astype(np.int32)).to(dev)
    src_info = torch.from_numpy(inp.src_info.astype(np.int32)).to(dev)
    ids = torch.from_numpy(inp.topk_ids.astype(np.int32)).to(dev)
    tw = torch.from_numpy(inp.topk_w).to(dev)
    out = torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def make_ctx(per_expert, epilogue_only=False, system_scope=False):
        return EpCombine(n_ranks=cfg.n_ranks, top_k=cfg.top_k,
                         max_tokens_per_rank=cfg.tokens_per_rank,
                         n_experts_per_device=cfg.n_experts_local, hidden_k=cfg.k, hidden_n=cfg.n,
                         my_rank=cfg.my_rank, msg_bytes=cfg.msg, dtype=cfg.dtype, device=dev,
                         per_expert_release=per_expert, epilogue_only=epilogue_only,
                         system_scope=system_scope)

    def time_local_c(ctx, warmup, steps):
        """Event time (ms) of each GEMM launch with the sink disabled: the
        kernel stores a local C [M][N] instead of scattering rows."""
        c = torch.empty((M, cfg.n), dtype=torch.bfloat16, device=dev)
        for _ in range(warmup):
            ctx.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws, p3_control=-1,
                             c_local=c, epoch=1)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            evs[i][0].record(stream)
            ctx.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws, p3_control=-1,
                             c_local=c, epoch=1)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        if ctx.query_error():
            raise RuntimeError("device error in the local-C launches")
        return np.array([e[0].elapsed_time(e[1]) for e in evs])

    def time_steps(ctx, settle_s, warmup, steps):
        """Settles the clocks, warms up, then times `steps` steps: returns the
        wall time per step and the per-launch GEMM and combine event times (ms)."""
        def one_step(ev=None):
            ctx.next_epoch()
            if ev is not None:
                ev[0].record(stream)
            ctx.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws)
            if ev is not None:
                ev[1].record(stream)
            ctx.combine(ids, tw, out)
            if ev is not None:
                ev[2].record(stream)

        n_settle = 0
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < settle_s:
            for _ in range(10):
                one_step()
            n_settle += 10
            torch.cuda.synchronize()
        for _ in range(warmup):
            one_step()
        torch.cuda.synchronize()
        if ctx.query_error():
            raise RuntimeError("device error during warmup")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one_step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        err = ctx.query_error()
        if err:
            raise RuntimeError(f"device error bits {err} in the timed steps")
        gemm = np.array([e[0].elapsed_time(e[1]) for e in evs])
        comb = np.array([e[1].elapsed_time(e[2]) for e in evs])
        return wall * 1e3 / steps, gemm, comb, n_settle

    ctx = make_ctx(False)
    print(f"[bench] settle {args.settle_s} s, warmup {args.warmup}", file=sys.stderr, flush=True)
    step_ms, gemm_ms, comb_ms, settle_steps = time_steps(ctx, args.settle_s, args.warmup,
                                                         args.steps)
    local_ms = epi_ms = None
    if not args.steps_only:
        print("[bench] sink disabled (local C)", file=sys.stderr, flush=True)
        local_ms = time_local_c(ctx, args.warmup, args.steps)
        # the same kernel with its K loop skipped: the sink epilogue alone (row
        # lookups, scatter stores, counts, elections), at the real shape
        print("[bench] epilogue-only launches (scatter time)", file=sys.stderr, flush=True)
        ctx_e = make_ctx(False, epilogue_only=True)
        _, epi_ms, _, _ = time_steps(ctx_e, min(args.settle_s, 0.3), args.warmup, args.steps)
        # the same two HBM-bound launches with the 256 MB MALL flushed before
        # each one (a 512 MiB fill outside the events): the combine rereads the
        # last step's slots under the same flag, the epilogue-only launch
        # rewrites them
        print("[bench] MALL-flushed combine and epilogue-only launches", file=sys.stderr, flush=True)
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        n_fl = max(5, min(args.steps, 20))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_fl)]
        for i in range(n_fl):
            flush_buf.fill_(i & 0xff)
            evs[i][0].record(stream)
            ctx.combine(ids, tw, out)
            evs[i][1].record(stream)
            flush_buf.fill_((i + 1) & 0xff)
            ctx_e.next_epoch()
            evs[i][2].record(stream)
            ctx_e.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws)
            evs[i][3].record(stream)
        torch.cuda.synchronize()
        if ctx.query_error() or ctx_e.query_error():
            raise RuntimeError("device error in the MALL-flushed launches")
        cold_comb_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        cold_epi_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
        del ctx_e, flush_buf
    del ctx

    n_nonempty = int(np.count_nonzero(inp.group_sizes()))
    gemm_b, scatter_b, combine_b = step_bytes(cfg, M, n_nonempty)
    flops = 2.0 * M * cfg.k * cfg.n
    g_avg = float(gemm_ms.mean())
    c_avg = float(comb_ms.mean())
    gemm_tflops = flops / (g_avg * 1e-3) / 1e12
    combine_gbs = combine_b / (c_avg * 1e-3) / 1e9
    e_avg = float(epi_ms.mean()) if epi_ms is not None else float("nan")
    sc_gbs = (scatter_b + combine_b) / ((e_avg + c_avg) * 1e-3) / 1e9
    peak = PEAK_TFLOPS[cfg.dtype]

    def pct(a):
        return {"p10": round(float(np.percentile(a, 10)) * 1e3, 2),
                "p50": round(float(np.percentile(a, 50)) * 1e3, 2),
                "p90": round(float(np.percentile(a, 90)) * 1e3, 2)}
    rec = {
        "metric": "grouped-GEMM+scatter TFLOP/s, combine GB/s, µs per EP-combine step (1 GPU)",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "steps": settle_steps},
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "ranks": cfg.n_ranks, "experts_global": cfg.n_experts_global,
                   "experts_local": cfg.n_experts_local, "tokens_per_rank": cfg.tokens_per_rank,
                   "top_k": cfg.top_k, "K": cfg.k, "N": cfg.n, "msg_bytes": cfg.msg,
                   "rows_M": M, "routing": cfg.routing, "parallelism": "single GPU share"},
        "gemm_scatter_tflops": round(gemm_tflops, 2),
        "gemm_scatter_us": round(g_avg * 1e3, 2),
        "combine_gbs": round(combine_gbs, 1),
        "combine_us": round(c_avg * 1e3, 2),
        "us_per_step": round(step_ms * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": stored_traffic(cfg),
                     "kernel": "gemm_scatter_bf16_kernel" if not fp8 else "gemm_scatter_fp8_kernel",
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": gemm_b},
        "combine_roofline": {"bound": "hbm", "achieved": round(combine_gbs, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(combine_gbs / PEAK_HBM_GBS, 4)},
        "event_us": {"gemm_scatter": pct(gemm_ms), "combine": pct(comb_ms)},
    }
    if not args.steps_only:
        # scatter time from the epilogue-only launches; bytes = scatter writes
        # + combine reads and writes
        rec["scatter_combine"] = {"bound": "hbm", "scatter_us": round(e_avg * 1e3, 2),
                                  "combine_us": round(c_avg * 1e3, 2),
                                  "bytes": scatter_b + combine_b, "achieved": round(sc_gbs, 1),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(sc_gbs / PEAK_HBM_GBS, 4)}
        rec["sink_vs_local_c"] = {"sink_us": round(g_avg * 1e3, 2),
                                  "local_c_us": round(float(local_ms.mean()) * 1e3, 2)}
        rec["event_us"]["epilogue_only"] = pct(epi_ms)
        rec["event_us"]["local_c"] = pct(local_ms)
        cc, ce = float(cold_comb_ms.mean()), float(cold_epi_ms.mean())
        cold_gbs = (scatter_b + combine_b) / ((cc + ce) * 1e-3) / 1e9
        rec["scatter_combine"]["mall_flushed"] = {
            "scatter_us": round(ce * 1e3, 2), "combine_us": round(cc * 1e3, 2),
            "combine_gbs": round(combine_b / (cc * 1e-3) / 1e9, 1),
            "achieved": round(cold_gbs, 1), "frac": round(cold_gbs / PEAK_HBM_GBS, 4)}
    if not args.no_up_proj and not args.steps_only and cfg.dtype == "bf16" and cfg.k % 128 == 0:
        # the expert FFN's first GEMM (hidden -> 2I, SwiGLU -> I), whose output
        # is this step's X: same rows and grouping, weights of its own
        from ep_synth import make_up_inputs
        print("[bench] up-projection + SwiGLU", file=sys.stderr, flush=True)
        x1_h, w1_h = make_up_inputs(cfg, M)
        x1 = torch.from_numpy(x1_h).view(torch.bfloat16).to(dev)
        w1 = torch.from_numpy(w1_h).view(torch.bfloat16).to(dev)
        del x1_h, w1_h
        h_out = torch.empty((M, cfg.k), dtype=torch.bfloat16, device=dev)
        ctx_u = make_ctx(False)
        for _ in range(max(args.warmup, 20)):
            ctx_u.up_swiglu(x1, w1, offsets, M, h_out)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            evs[i][0].record(stream)
            ctx_u.up_swiglu(x1, w1, offsets, M, h_out)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        if ctx_u.query_error():
            raise RuntimeError("device error in the up-projection launches")
        u_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        u_flops = 2.0 * M * cfg.n * 2 * cfg.k
        u_tflops = u_flops / (float(u_ms.mean()) * 1e-3) / 1e12
        rec["up_swiglu"] = {
            "shape": {"rows_M": M, "hidden": cfg.n, "I": cfg.k, "experts_local": cfg.n_experts_local},
            "us": round(float(u_ms.mean()) * 1e3, 2), "event_us": pct(u_ms),
            "tflops": round(u_tflops, 2),
            "roofline": {"bound": "mfma", "achieved": round(u_tflops, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(u_tflops / peak, 4),
                         "algorithmic_flops_per_launch": u_flops}}
        del ctx_u, x1, w1, h_out
    if not args.no_per_expert and not args.steps_only:
        # per-expert completion (every count word its own release store, the
        # combine acquiring each) beside the rank-level election: same inputs
        print("[bench] per-expert completion variant", file=sys.stderr, flush=True)
        ctx2 = make_ctx(True)
        p_ms, p_gemm, p_comb, _ = time_steps(ctx2, min(args.settle_s, 0.3), args.warmup,
                                             args.steps)
        del ctx2
        rec["per_expert_completion"] = {
            "us_per_step": round(p_ms * 1e3, 2),
            "gemm_scatter_us": round(float(p_gemm.mean()) * 1e3, 2),
            "combine_us": round(float(p_comb.mean()) * 1e3, 2),
            "release_stores_per_step": cfg.n_experts_local * cfg.n_ranks,
            "rank_level_release_stores_per_step": cfg.n_ranks}
    if not args.no_per_expert and not args.steps_only:
        # the pages' system-scope publication (the scope a multi-GPU step needs)
        # beside the agent scope a single GPU needs: same inputs
        print("[bench] system-scope variant", file=sys.stderr, flush=True)
        ctx3 = make_ctx(False, system_scope=True)
        s_ms, s_gemm, s_comb, _ = time_steps(ctx3, min(args.settle_s, 0.3), args.warmup,
                                             args.steps)
        del ctx3
        rec["system_scope"] = {
            "us_per_step": round(s_ms * 1e3, 2),
            "gemm_scatter_us": round(float(s_gemm.mean()) * 1e3, 2),
            "combine_us": round(float(s_comb.mean()) * 1e3, 2)}
    if not args.steps_only:
        # local grouping of the routing (upstream input preparation, outside the
        # step): event time of ep_group_local_picks at this workload's routing
        print("[bench] local grouping", file=sys.stderr, flush=True)
        ctx_g = make_ctx(False)
        g_off = torch.empty(cfg.n_experts_local * cfg.n_ranks + 1, dtype=torch.int32, device=dev)
        g_src = torch.empty((ids.numel(), 2), dtype=torch.int32, device=dev)
        for _ in range(args.warmup):
            ctx_g.group(ids, offsets=g_off, src_info=g_src)
        torch.cuda.synchronize()
        g_ms = []
        for _ in range(max(args.steps, 5)):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            ctx_g.group(ids, offsets=g_off, src_info=g_src)
            s1.record()
            g_ms.append((s0, s1))
        torch.cuda.synchronize()
        if not torch.equal(g_off.cpu(), offsets.cpu()):
            raise RuntimeError("ep_group_local_picks disagrees with the generator's layout")
        rec["local_grouping_us"] = pct([a.elapsed_time(b) for a, b in g_ms])
        del ctx_g, g_off, g_src
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a CPU sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of one EP-combine step on one MI355X.

A step is one pass of the whole path on one batch of synthetic input: the
grouped GEMM with the in-epilogue row scatter and fused completion signals
(ep_grouped_gemm_scatter) followed by the consumer combine (ep_combine_reduce),
both through the C ABI, inputs resident in HBM.  The grouped row layout comes
from the library's own grouping of the routing (ep_group_local_picks), done
once before timing (it stands for the upstream dispatch).  Prints one JSON
line: the headline workload (DeepSeek-V3-shaped prefill by default) at the top
level, and every named workload under "workloads", each with its own roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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
    "bf16": ["gemm_scatter.hip", "gemm_bf16.h", "gemm_common.h", "ep_device.h", "ep_kernels.h"],
    "fp8": ["gemm_scatter_fp8.hip", "gemm_common.h", "ep_device.h", "ep_kernels.h"],
}
COPY_PROBE_BYTES = 1 << 30
ALL_WORKLOADS = ["deepseek_prefill", "deepseek_decode", "qwen3_moe", "skewed_fp8", "tiny"]
TILE_KERNEL = {0: "256x256", 1: "128x128", 2: "256x128", 3: "64x128 (small row groups)",
               4: "128x128 with send waves", 5: "128x128, sink in the MFMA waves"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup: the GPU takes tens of "
                         "milliseconds of sustained load to reach its steady clocks")
    ap.add_argument("--config", default="deepseek_prefill", help="headline workload")
    ap.add_argument("--workloads", default="all",
                    help="comma-separated further workloads timed after the headline one "
                         "('all': every named workload, 'none': only the headline)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens per rank in the oracle's timed sample (0: all of them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--steps-only", action="store_true",
                    help="time the EP-combine steps of the headline workload alone: no other "
                         "workloads and no local-C, epilogue-only or variant launches (used for "
                         "the hardware-counter runs, so every launch of the GEMM kernel is a "
                         "step's)")
    ap.add_argument("--no-up-proj", action="store_true",
                    help="skip the up-projection + SwiGLU GEMM measurement")
    ap.add_argument("--no-per-expert", action="store_true",
                    help="skip timing the per-expert completion and system-scope variants")
    ap.add_argument("--w-layout", choices=["auto", "row_major", "slice_major"], default="auto",
                    help="layout of the down-projection weights: row-major [E][N][K], or "
                         "slice-major [E][K/64][N][64] (bf16; packed once, outside the timed "
                         "region); auto: slice-major where the GEMM runs on the decode tile")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the HBM byte counters)")
    return ap.parse_args()


def gpu_state():
    """Shader clock (the current DPM level), board power and power cap of the
    GPU as its driver reports them in sysfs, or {} where they are not readable.
    Read right after a timed region: under sustained MFMA load the GPU runs at
    its power cap, below the clock the published peaks assume."""
    import glob
    st = {}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))[:1]:
        try:
            cur = [ln for ln in open(f).read().split("\n") if ln.strip().endswith("*")]
            if cur:
                st["sclk_mhz"] = float(cur[0].split()[1].lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            pass
    for name, key in (("power1_input", "power_w"), ("power1_average", "power_w"),
                      ("power1_cap", "power_cap_w")):
        for f in sorted(glob.glob(f"/sys/class/drm/card*/device/hwmon/hwmon*/{name}"))[:1]:
            try:
                st.setdefault(key, int(open(f).read()) / 1e6)
            except (OSError, ValueError):
                pass
    return st


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
    """Algorithmic bytes: GEMM (each non-empty expert's W_e, X, the sent rows,
    fp8 scales), scatter (the sent rows) and combine (slot reads, output
    writes, routing ids and weights)."""
    elt = 1 if cfg.dtype == "fp8" else 2
    K, N, R, T, k = cfg.k, cfg.n, cfg.n_ranks, cfg.tokens_per_rank, cfg.top_k
    scales = 0
    if cfg.dtype == "fp8":
        scales = M * (K // 128) * 4 + n_nonempty * (N // 128) * (K // 128) * 4
    gemm = n_nonempty * K * N * elt + M * K * elt + M * 2 * N + scales
    scatter = M * 2 * N
    combine = M * 2 * N + R * T * 2 * N + R * T * k * 8
    return gemm, scatter, combine


def gemm_roofline(cfg, M, flops, gemm_b, t_s):
    """Roofline of the GEMM launch: the bound is the larger of the MFMA time
    (flops / dtype peak) and the HBM time (algorithmic bytes / 8 TB/s);
    achieved and peak are in that bound's unit."""
    peak = PEAK_TFLOPS[cfg.dtype]
    t_mfma = flops / (peak * 1e12)
    t_hbm = gemm_b / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = flops / t_s / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
             "frac": round(ach / peak, 4)}
    else:
        ach = gemm_b / t_s / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(ach / PEAK_HBM_GBS, 4)}
    r.update({"roofline_us": round(max(t_mfma, t_hbm) * 1e6, 2),
              "arithmetic_intensity_flop_per_byte": round(flops / gemm_b, 1),
              "ridge_flop_per_byte": round(peak * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
              "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": gemm_b})
    return r


def host_cpu():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline(inp, tokens):
    """Times the oracle on the whole step of the same workload (or a token
    prefix of every rank): grouping, binary32 GEMM, scatter, counts, combine.
    The X rows of the oracle's picks are drawn before the clock starts."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    model, cores = host_cpu()
    cfg = inp.cfg
    S = cfg.tokens_per_rank if tokens <= 0 else min(tokens, cfg.tokens_per_rank)
    ids, tw = inp.topk_ids[:, :S], inp.topk_w[:, :S]
    off, src = O.group_local_picks(ids, cfg.n_experts_local, cfg.my_rank)
    x, xs = inp.rows(O.row_picks(off, src, cfg.n_ranks))
    t0 = time.perf_counter()
    res = O.run_step(topk_ids=ids, topk_w=tw, x=x, x_scale=xs, w=inp.w, w_scale=inp.w_scale,
                     n_ranks=cfg.n_ranks, n_experts_per_device=cfg.n_experts_local,
                     top_k=cfg.top_k, msg_bytes=cfg.msg, max_tokens_per_rank=S,
                     my_rank=cfg.my_rank, dtype=cfg.dtype)
    dt = time.perf_counter() - t0
    Ms = int(res["offsets"][-1])
    flops = 2.0 * Ms * cfg.k * cfg.n
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "cpu_model": model, "blas_threads": blas, "kind": "oracle",
            "us_per_step": round(dt * 1e6, 1),
            "sample": (f"all {S} tokens per rank" if S == cfg.tokens_per_rank else
                       f"first {S} of {cfg.tokens_per_rank} tokens per rank") +
                      f": {Ms} rows, whole step (grouping, binary32 GEMM, scatter, counts, "
                      f"combine), {dt:.2f} s"}


def practical_ceiling(torch, dev, stream, cfg, offsets, src_info, M, scatter_b, combine_b,
                      scatter_ms, combine_ms, reps=20):
    """This machine's own rates for the access patterns of the scatter and the
    combine, with library kernels (torch): a sequential fill of the scatter's
    bytes, a fill of 512-byte pieces at exactly the slots and columns the sink
    writes (index_fill_ over the receive area), and a plain copy of the
    combine's bytes.  The practical time of scatter + combine is the scattered
    fill's time plus the copy's; `frac` compares it with the measured one."""
    R, T, k, N, msg = cfg.n_ranks, cfg.tokens_per_rank, cfg.top_k, cfg.n, cfg.msg
    if N % 256 or msg % 512:
        return None

    def timed(fn):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # piece index of every (row, 256-column block): rank rk's buffer follows rank rk-1's
    rows = torch.arange(M, dtype=torch.int32, device=dev)
    rk = ((torch.searchsorted(offsets, rows, right=True) - 1) % R).to(torch.int64)
    slot = rk * (T * k) + src_info[:M, 0].to(torch.int64) * k + src_info[:M, 1].to(torch.int64)
    per_slot = msg // 512
    idx = (slot[:, None] * per_slot + torch.arange(N // 256, device=dev)[None, :]).reshape(-1)
    area = torch.empty((R * T * k * per_slot, 256), dtype=torch.bfloat16, device=dev)
    seq = torch.empty(scatter_b // 2, dtype=torch.bfloat16, device=dev)
    fill_ms = timed(lambda: seq.fill_(1.0))
    scat_ms = timed(lambda: area.index_fill_(0, idx, 1.0))
    del area, seq
    src = torch.empty(combine_b // 4, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src))
    del src, dst
    t_prac = scat_ms + copy_ms
    return {"fill_gbs": round(scatter_b / (fill_ms * 1e-3) / 1e9, 1),
            "scattered_512b_fill_gbs": round(scatter_b / (scat_ms * 1e-3) / 1e9, 1),
            "copy_gbs": round(combine_b / (copy_ms * 1e-3) / 1e9, 1),
            "practical_us": round(t_prac * 1e3, 2),
            "practical_gbs": round((scatter_b + combine_b) / (t_prac * 1e-3) / 1e9, 1),
            "practical_frac_of_8tbs": round((scatter_b + combine_b) / (t_prac * 1e-3) / 8e12, 4),
            "frac": round(t_prac / (scatter_ms + combine_ms), 4)}


def send_waves_short_k(cfg, args, dev, stream, K=256):
    """The same routing with K = 256 (a probe shape, not a named workload):
    four K slices per tile, so a tile's epilogue weighs about as much as its K
    loop and the send waves have something to hide.  GEMM + sink event time
    (median of `steps` launches) of the default kernel, the send-wave kernel
    and the same kernel with the sink inside its MFMA waves."""
    import numpy as np
    import torch
    from ep_synth import make_inputs
    from grouped_gemm_scatter_amd import EpCombine
    c2 = cfg.replace(k=K)
    inp = make_inputs(c2)
    res = {"K": K}
    for key, kw in [("default", {}), ("send_waves_4", {"send_waves": 4}),
                    ("sink_in_mfma_waves", {"send_tile": True})]:
        ctx = EpCombine(n_ranks=c2.n_ranks, top_k=c2.top_k, max_tokens_per_rank=c2.tokens_per_rank,
                        n_experts_per_device=c2.n_experts_local, hidden_k=c2.k, hidden_n=c2.n,
                        my_rank=c2.my_rank, msg_bytes=c2.msg, dtype=c2.dtype, device=dev, **kw)
        ids = torch.from_numpy(inp.topk_ids.astype(np.int32)).to(dev)
        off, src = ctx.group(ids)
        M = int(off[-1].item())
        rows = torch.arange(M, dtype=torch.int32, device=dev)
        rk = ((torch.searchsorted(off, rows, right=True) - 1) % c2.n_ranks).to(torch.int64)
        picks = torch.stack([rk, src[:M, 0].long(), src[:M, 1].long()], 1).cpu().numpy()
        x = torch.from_numpy(inp.rows(picks)[0]).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(inp.w).view(torch.bfloat16).to(dev)
        for _ in range(max(args.warmup, 10)):
            ctx.next_epoch()
            ctx.gemm_scatter(x, w, off, src, M)
        evs = []
        for _ in range(max(args.steps, 20)):
            ctx.next_epoch()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ctx.gemm_scatter(x, w, off, src, M)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        if ctx.query_error():
            raise RuntimeError("device error in the short-K send-wave launches")
        res[key + "_us"] = round(float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3, 2)
        res["rows_M"] = M
        ctx.close()
        del ctx, x, w
    return res


def pct(a):
    return {"p10": round(float(np.percentile(a, 10)) * 1e3, 2),
            "p50": round(float(np.percentile(a, 50)) * 1e3, 2),
            "p90": round(float(np.percentile(a, 90)) * 1e3, 2)}


def measure(cfg, args, headline):
    """Times one workload; returns its record."""
    import torch

    from ep_synth import make_inputs
    from grouped_gemm_scatter_amd import EpCombine

    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg)
    fp8 = cfg.dtype == "fp8"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    layout = {"slice_major": False}

    def make_ctx(per_expert=False, epilogue_only=False, system_scope=False, slice_major=None,
                 device_epoch=False, **extra):
        return EpCombine(n_ranks=cfg.n_ranks, top_k=cfg.top_k,
                         max_tokens_per_rank=cfg.tokens_per_rank,
                         n_experts_per_device=cfg.n_experts_local, hidden_k=cfg.k, hidden_n=cfg.n,
                         my_rank=cfg.my_rank, msg_bytes=cfg.msg, dtype=cfg.dtype, device=dev,
                         per_expert_release=per_expert, epilogue_only=epilogue_only,
                         system_scope=system_scope,
                         w_slice_major=layout["slice_major"] if slice_major is None
                         else slice_major, device_epoch=device_epoch, **extra)

    ctx = make_ctx()
    ids = torch.from_numpy(inp.topk_ids.astype(np.int32)).to(dev)
    tw = torch.from_numpy(inp.topk_w).to(dev)
    # the library's own grouping of the routing; X rows of the picks it lists
    offsets, src_info = ctx.group(ids)
    M = int(offsets[-1].item())
    rows = torch.arange(M, dtype=torch.int32, device=dev)
    rk = ((torch.searchsorted(offsets, rows, right=True) - 1) % cfg.n_ranks).to(torch.int64)
    picks = torch.stack([rk, src_info[:M, 0].to(torch.int64), src_info[:M, 1].to(torch.int64)],
                        dim=1).cpu().numpy()
    x_h, xs_h = inp.rows(picks)
    x = torch.from_numpy(x_h).view(torch.uint8 if fp8 else torch.bfloat16).to(dev) if M else None
    xs = torch.from_numpy(xs_h).to(dev) if fp8 and M else None
    w = torch.from_numpy(inp.w).view(torch.uint8 if fp8 else torch.bfloat16).to(dev)
    ws = torch.from_numpy(inp.w_scale).to(dev) if fp8 else None
    out = torch.empty((cfg.n_ranks, cfg.tokens_per_rank, cfg.n), dtype=torch.bfloat16, device=dev)
    del rows, rk
    w_row = w
    if not fp8 and (args.w_layout == "slice_major" or
                    (args.w_layout == "auto" and ctx.gemm_tile(M)[0] == 3)):
        # weights re-laid once, as at weight load (not part of a step)
        layout["slice_major"] = True
        ctx.close()
        ctx = make_ctx()
        w = ctx.pack_weights(w_row)
        torch.cuda.synchronize()

    def time_local_c(c_ctx, warmup, steps):
        """Event time (ms) of each GEMM launch with the sink disabled: the
        kernel stores a local C [M][N] instead of scattering rows."""
        c = torch.empty((max(M, 1), cfg.n), dtype=torch.bfloat16, device=dev)
        for _ in range(warmup):
            c_ctx.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws, p3_control=-1,
                               c_local=c, epoch=1)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            evs[i][0].record(stream)
            c_ctx.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws, p3_control=-1,
                               c_local=c, epoch=1)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        if c_ctx.query_error():
            raise RuntimeError("device error in the local-C launches")
        return np.array([e[0].elapsed_time(e[1]) for e in evs])

    state = {}

    def time_steps(s_ctx, settle_s, warmup, steps, fused=False):
        """Settles the clocks, warms up, then times `steps` steps: returns the
        wall time per step and the per-launch GEMM and combine event times (ms),
        each recorded on the stream the launches go to (fused: one launch, its
        time in the GEMM column, combine 0)."""
        def one_step(ev=None):
            s_ctx.next_epoch()
            if ev is not None:
                ev[0].record(stream)
            if fused:
                s_ctx.gemm_scatter_combine(x, w, offsets, src_info, M, ids, tw, out,
                                           x_scale=xs, w_scale=ws)
            else:
                s_ctx.gemm_scatter(x, w, offsets, src_info, M, x_scale=xs, w_scale=ws)
            if ev is not None:
                ev[1].record(stream)
            if not fused:
                s_ctx.combine(ids, tw, out)
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
        if s_ctx.query_error():
            raise RuntimeError("device error during warmup")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one_step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        state.clear()
        state.update(gpu_state())
        err = s_ctx.query_error()
        if err:
            raise RuntimeError(f"device error bits {err} in the timed steps")
        gemm = np.array([e[0].elapsed_time(e[1]) for e in evs])
        comb = np.array([e[1].elapsed_time(e[2]) for e in evs])
        return wall * 1e3 / steps, gemm, comb, n_settle

    settle = args.settle_s if headline else min(args.settle_s, 0.5)
    print(f"[bench] {cfg.name}: settle {settle} s, warmup {args.warmup}, {args.steps} steps",
          file=sys.stderr, flush=True)
    step_ms, gemm_ms, comb_ms, settle_steps = time_steps(ctx, settle, args.warmup, args.steps)
    step_state = dict(state)
    extras = not args.steps_only
    fused_ms = fused_ev = None
    if extras:
        # the same step as one launch (ep_grouped_gemm_scatter_combine: the
        # consumer runs in the GEMM's grid)
        fused_ms, fused_ev, _, _ = time_steps(ctx, min(settle, 0.3), args.warmup, args.steps,
                                              fused=True)
    local_ms = epi_ms = None
    if extras:
        print(f"[bench] {cfg.name}: sink disabled (local C)", file=sys.stderr, flush=True)
        local_ms = time_local_c(ctx, args.warmup, args.steps)
        # the same kernel with its K loop skipped: the sink epilogue alone (row
        # lookups, scatter stores, counts, elections), at the real shape
        print(f"[bench] {cfg.name}: epilogue-only launches (scatter time)", file=sys.stderr,
              flush=True)
        ctx_e = make_ctx(epilogue_only=True)
        _, epi_ms, _, _ = time_steps(ctx_e, min(args.settle_s, 0.3), args.warmup, args.steps)

    n_nonempty = int(np.count_nonzero(np.diff(
        offsets.cpu().numpy()[:: cfg.n_ranks][: cfg.n_experts_local + 1])))
    gemm_b, scatter_b, combine_b = step_bytes(cfg, M, n_nonempty)
    flops = 2.0 * M * cfg.k * cfg.n
    g_avg, c_avg = float(gemm_ms.mean()), float(comb_ms.mean())
    tile_kind, tile_m, tile_n = ctx.gemm_tile(M)
    roof = gemm_roofline(cfg, M, flops, gemm_b, g_avg * 1e-3)
    roof["traffic"] = stored_traffic(cfg)
    tile_name = (f"up to {tile_m}x{tile_n} (an expert's rows spread evenly over its row tiles)"
                 if tile_kind == 0 and not fp8 else TILE_KERNEL.get(tile_kind))
    roof["kernel"] = (("gemm_scatter_fp8_kernel" if fp8 else
                       "gemm_scatter_bf16_decode_kernel" if tile_kind == 3 else
                       "gemm_scatter_bf16_kernel") + f", {tile_name} tile")
    if "sclk_mhz" in step_state and roof["bound"] == "mfma":
        # the same peak at the clock the GPU ran at (the published one assumes 2400 MHz)
        roof["peak_at_measured_clock"] = round(roof["peak"] * step_state["sclk_mhz"] / 2400.0, 1)
    combine_gbs = combine_b / (c_avg * 1e-3) / 1e9
    rec = {
        "workload": cfg.name,
        "config": {"workload": cfg.name, "ranks": cfg.n_ranks,
                   "experts_global": cfg.n_experts_global, "experts_local": cfg.n_experts_local,
                   "tokens_per_rank": cfg.tokens_per_rank, "top_k": cfg.top_k, "K": cfg.k,
                   "N": cfg.n, "msg_bytes": cfg.msg, "rows_M": M, "routing": cfg.routing,
                   "dtype": cfg.dtype, "experts_nonempty": n_nonempty,
                   "parallelism": "single GPU share"},
        "us_per_step": round(step_ms * 1e3, 2),
        "step_tflops": round(flops / (step_ms * 1e-3) / 1e12, 3),
        "gemm_scatter_us": round(g_avg * 1e3, 2),
        "gemm_scatter_tflops": round(flops / (g_avg * 1e-3) / 1e12, 2),
        "combine_us": round(c_avg * 1e3, 2),
        "combine_gbs": round(combine_gbs, 1),
        "roofline": roof,
        "combine_roofline": {"bound": "hbm", "achieved": round(combine_gbs, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(combine_gbs / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes_per_launch": combine_b},
        "event_us": {"gemm_scatter": pct(gemm_ms), "combine": pct(comb_ms)},
        "gpu_state": step_state,
        "settle": {"seconds": settle, "steps": settle_steps},
    }
    rec["config"]["w_layout"] = "slice_major" if layout["slice_major"] else "row_major"
    if extras:
        # the step captured once in a HIP graph and replayed (epoch in device
        # memory, advanced by the graph itself): no host work per step
        print(f"[bench] {cfg.name}: graph replay", file=sys.stderr, flush=True)
        g_ctx = make_ctx(device_epoch=True)

        def g_step():
            g_ctx.step(x, w, offsets, src_info, M, ids, tw, out, x_scale=xs, w_scale=ws)

        g_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g_step()
        for _ in range(max(args.warmup, 5)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        g_us = (time.perf_counter() - t0) * 1e6 / args.steps
        if g_ctx.query_error():
            raise RuntimeError("device error in the graph replays")
        rec["graph_step"] = {"us_per_step": round(g_us, 2),
                             "two_launch_us_per_step": round(step_ms * 1e3, 2)}
        del graph, g_ctx
    if extras and layout["slice_major"]:
        # the same steps reading the row-major weights, for comparison
        print(f"[bench] {cfg.name}: row-major weights", file=sys.stderr, flush=True)
        r_ctx = make_ctx(slice_major=False)
        w_packed, w = w, w_row
        r_ms, r_gemm, _, _ = time_steps(r_ctx, min(args.settle_s, 0.3), args.warmup, args.steps)
        w = w_packed
        r_ctx.close()
        del r_ctx
        rec["row_major_w"] = {"us_per_step": round(r_ms * 1e3, 2),
                              "gemm_scatter_us": round(float(r_gemm.mean()) * 1e3, 2)}
    if extras:
        rec["event_us"]["fused_step"] = pct(fused_ev)
        rec["fused_step"] = {"us_per_step": round(fused_ms * 1e3, 2),
                             "launch_us": round(float(fused_ev.mean()) * 1e3, 2),
                             "two_launch_us_per_step": round(step_ms * 1e3, 2),
                             "gemm_plus_combine_us": round((g_avg + c_avg) * 1e3, 2)}
    if cfg.name == "tiny":
        rec["note"] = "launch-bound: a few kilobytes of work per launch"
    if extras:
        e_avg = float(epi_ms.mean())
        sc_gbs = (scatter_b + combine_b) / ((e_avg + c_avg) * 1e-3) / 1e9
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
    if extras and headline:
        # the two HBM-bound launches with the 256 MB MALL flushed before each
        # one (a 512 MiB fill outside the events): the combine rereads the last
        # step's slots under the same flag, the epilogue-only launch rewrites them
        print("[bench] MALL-flushed combine and epilogue-only launches", file=sys.stderr,
              flush=True)
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
        cc = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        ce = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
        cold_gbs = (scatter_b + combine_b) / ((cc + ce) * 1e-3) / 1e9
        rec["scatter_combine"]["mall_flushed"] = {
            "scatter_us": round(ce * 1e3, 2), "combine_us": round(cc * 1e3, 2),
            "combine_gbs": round(combine_b / (cc * 1e-3) / 1e9, 1),
            "achieved": round(cold_gbs, 1), "frac": round(cold_gbs / PEAK_HBM_GBS, 4)}
        del flush_buf
        rec["scatter_combine"]["practical"] = practical_ceiling(
            torch, dev, stream, cfg, offsets, src_info, M, scatter_b, combine_b, e_avg, c_avg)
    if extras:
        del ctx_e
    if extras and not args.no_up_proj and (headline or fp8) and cfg.k % 128 == 0:
        # the expert FFN's first GEMM (hidden -> 2I, SwiGLU -> I), whose output
        # is this step's X: same rows and grouping, inputs of its own (fp8:
        # block-scaled operands, H re-quantised with its row-block scales)
        print(f"[bench] {cfg.name}: up-projection + SwiGLU", file=sys.stderr, flush=True)
        if fp8:
            x1_h, x1s_h = inp.up_rows(picks)
            w1_h, w1s_h = inp.up_weights()
            x1, x1s = torch.from_numpy(x1_h).to(dev), torch.from_numpy(x1s_h).to(dev)
            w1, w1s = torch.from_numpy(w1_h).to(dev), torch.from_numpy(w1s_h).to(dev)
            h_out = torch.empty((M, cfg.k), dtype=torch.uint8, device=dev)
            h_scale = torch.empty((M, cfg.k // 128), dtype=torch.float32, device=dev)

            def up():
                ctx.up_swiglu_fp8(x1, x1s, w1, w1s, offsets, M, h_out, h_scale)
        else:
            x1 = torch.from_numpy(inp.up_rows(picks)).view(torch.bfloat16).to(dev)
            w1 = torch.from_numpy(inp.up_weights()).view(torch.bfloat16).to(dev)
            h_out = torch.empty((M, cfg.k), dtype=torch.bfloat16, device=dev)

            def up():
                ctx.up_swiglu(x1, w1, offsets, M, h_out)
        for _ in range(max(args.warmup, 20)):
            up()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            evs[i][0].record(stream)
            up()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        if ctx.query_error():
            raise RuntimeError("device error in the up-projection launches")
        u_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        u_flops = 2.0 * M * cfg.n * 2 * cfg.k
        u_tflops = u_flops / (float(u_ms.mean()) * 1e-3) / 1e12
        peak = PEAK_TFLOPS[cfg.dtype]
        rec["up_swiglu"] = {
            "shape": {"rows_M": M, "hidden": cfg.n, "I": cfg.k,
                      "experts_local": cfg.n_experts_local, "dtype": cfg.dtype},
            "us": round(float(u_ms.mean()) * 1e3, 2), "event_us": pct(u_ms),
            "tflops": round(u_tflops, 2),
            "roofline": {"bound": "mfma", "achieved": round(u_tflops, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(u_tflops / peak, 4),
                         "algorithmic_flops_per_launch": u_flops}}
        del x1, w1, h_out
    if extras and headline and not fp8:
        # dedicated send waves ("EpiloguePeerSink" SendWarps): the 128 x 128
        # kernel with 4 send waves beside the same kernel with the sink inside
        # its MFMA waves, same inputs
        rec["send_waves"] = {}
        for key, kw in [("send_waves_4", {"send_waves": 4}),
                        ("sink_in_mfma_waves", {"send_tile": True})]:
            print(f"[bench] {key}", file=sys.stderr, flush=True)
            v_ctx = make_ctx(**kw)
            v_ms, v_gemm, v_comb, _ = time_steps(v_ctx, min(args.settle_s, 0.3), args.warmup,
                                                 args.steps)
            del v_ctx
            rec["send_waves"][key] = {"us_per_step": round(v_ms * 1e3, 2),
                                      "gemm_scatter_us": round(float(v_gemm.mean()) * 1e3, 2),
                                      "gemm_event_us": pct(v_gemm)}
        rec["send_waves"]["tile"] = "128x128, 8 MFMA waves, three K-slice stages"
        rec["send_waves"]["short_k"] = send_waves_short_k(cfg, args, dev, stream)
    if extras and headline and not args.no_per_expert:
        # per-expert completion (every count word its own release store, the
        # combine acquiring each) and the pages' system-scope publication (the
        # scope a multi-GPU step needs), beside the rank-level election at agent
        # scope: same inputs
        for key, kw in [("per_expert_completion", {"per_expert": True}),
                        ("system_scope", {"system_scope": True})]:
            print(f"[bench] {key} variant", file=sys.stderr, flush=True)
            v_ctx = make_ctx(**kw)
            v_ms, v_gemm, v_comb, _ = time_steps(v_ctx, min(args.settle_s, 0.3), args.warmup,
                                                 args.steps)
            del v_ctx
            rec[key] = {"us_per_step": round(v_ms * 1e3, 2),
                        "gemm_scatter_us": round(float(v_gemm.mean()) * 1e3, 2),
                        "combine_us": round(float(v_comb.mean()) * 1e3, 2)}
        rec["per_expert_completion"].update({
            "release_stores_per_step": cfg.n_experts_local * cfg.n_ranks,
            "rank_level_release_stores_per_step": cfg.n_ranks})
    if extras:
        # local grouping of the routing (upstream input preparation, outside
        # the step): event time of ep_group_local_picks at this routing
        print(f"[bench] {cfg.name}: local grouping", file=sys.stderr, flush=True)
        g_off = torch.empty_like(offsets)
        g_src = torch.empty_like(src_info)
        for _ in range(args.warmup):
            ctx.group(ids, offsets=g_off, src_info=g_src)
        torch.cuda.synchronize()
        g_ev = []
        for _ in range(max(args.steps, 5)):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            ctx.group(ids, offsets=g_off, src_info=g_src)
            s1.record(stream)
            g_ev.append((s0, s1))
        torch.cuda.synchronize()
        if not torch.equal(g_off, offsets):
            raise RuntimeError("ep_group_local_picks is not deterministic")
        rec["local_grouping_us"] = pct([a.elapsed_time(b) for a, b in g_ev])
        del g_off, g_src
    if extras and headline:
        # dispatch side (outside the step, like the grouping): every local
        # pick's token row gathered into the grouped X1 of the up-projection
        print(f"[bench] {cfg.name}: dispatch rows", file=sys.stderr, flush=True)
        toks = torch.from_numpy(inp.tokens()).view(torch.bfloat16).to(dev)
        x1d = torch.empty((max(M, 1), cfg.n), dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup):
            ctx.dispatch(toks, offsets, src_info, M, x1d)
        d_ev = []
        for _ in range(max(args.steps, 5)):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            ctx.dispatch(toks, offsets, src_info, M, x1d)
            s1.record(stream)
            d_ev.append((s0, s1))
        torch.cuda.synchronize()
        if ctx.query_error():
            raise RuntimeError("device error in the dispatch launches")
        d_ms = np.array([a.elapsed_time(b) for a, b in d_ev])
        d_bytes = 2 * M * 2 * cfg.n          # each row read from its token and written
        rec["dispatch"] = {"us": round(float(d_ms.mean()) * 1e3, 2), "event_us": pct(d_ms),
                           "bytes": d_bytes,
                           "gbs": round(d_bytes / (float(d_ms.mean()) * 1e-3) / 1e9, 1),
                           "frac_of_8tbs": round(d_bytes / (float(d_ms.mean()) * 1e-3) / 8e12, 4)}
        del toks, x1d
    del ctx, x, w, xs, ws, out, offsets, src_info, ids, tw
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print(f"[bench] {cfg.name}: timing the oracle on the host", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    return rec


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the EP combine and runs on one GPU only; "
              "on more GPUs each would run the same step on its own expert slice, with the "
              "receive buffers of the other ranks mapped from their GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch

    from ep_synth import config_by_name

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = config_by_name(args.config)
    head = measure(cfg, args, headline=True)
    others = []
    if not args.steps_only and args.workloads != "none":
        names = ALL_WORKLOADS if args.workloads == "all" else args.workloads.split(",")
        others = [n for n in names if n != cfg.name]
    workloads = {cfg.name: head}
    for name in others:
        workloads[name] = measure(config_by_name(name), args, headline=False)

    flops = 2.0 * head["config"]["rows_M"] * cfg.k * cfg.n
    rec = {
        "metric": "grouped-GEMM+scatter TFLOP/s, combine GB/s, µs per EP-combine step (1 GPU)",
        "value": round(flops / (head["us_per_step"] * 1e-6) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
    }
    rec.update({k: v for k, v in head.items() if k != "workload"})
    if "cpu_baseline" in head:
        rec["cpu_baseline"] = head["cpu_baseline"]
    if len(workloads) > 1:
        rec["workloads"] = {n: {k: v for k, v in r.items() if k not in ("workload",)}
                            for n, r in workloads.items() if n != cfg.name}
        rec["summary"] = {n: {"us_per_step": r["us_per_step"],
                              "gemm_us": r["gemm_scatter_us"],
                              "gemm_bound": r["roofline"]["bound"],
                              "gemm_frac": r["roofline"]["frac"],
                              "combine_frac": r["combine_roofline"]["frac"],
                              "scatter_combine_frac": r.get("scatter_combine", {}).get("frac"),
                              "fused_us_per_step": r.get("fused_step", {}).get("us_per_step")}
                          for n, r in workloads.items()}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

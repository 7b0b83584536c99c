"""Seeded input generator (numpy + torch CPU casts; no GPU, no combine arithmetic).

Recipe, for a configuration with R ranks, E_g global / E_l local experts,
T tokens per rank, top_k picks, GEMM dims K x N and seed s:

* routing, drawn from ``default_rng(SeedSequence([s, 0]))``:
  - uniform: i.i.d. U(0,1) scores over the E_g experts for every (rank, token);
    the top_k highest scores are the picks, in descending score order (a
    uniformly random set of top_k distinct experts);
  - zipf: expert g has popularity (pi(g)+1)^(-zipf_s) for a random permutation
    pi; the n_forced_empty local experts of lowest popularity get popularity 0;
    picks are top_k distinct experts drawn without replacement in proportion
    to popularity (Gumbel-top-k), in descending key order;
  - routing weights: softmax (in float64, stored float32) of N(0,1) logits over
    the top_k picks of each token.
* dispatched rows: the picks whose expert lies in this GPU's slice
  [my_rank*E_l, (my_rank+1)*E_l) are laid out grouped by local expert e and,
  inside a group, sorted by (rk, t, k).  ``offsets[e*R + rk]`` is the first row
  of the (expert e, source rank rk) run, ``offsets[E_l*R]`` = M, and
  ``src_info[m] = (t, k)`` is the token index on its owner rank and its pick
  position.  This layout is the output of the upstream dispatch and the input
  of the grouped GEMM.
* X rows: N(0,1) float32 from ``SeedSequence([s, 1, chunk])`` per 4096-row chunk.
* W_e: N(0,1)/sqrt(K) float32 from ``SeedSequence([s, 2, e])``, stored
  K-contiguous as ``[E_l][N][K]`` (the logical K x N matrix, transposed).
* bf16: round-to-nearest-even cast of the float32 draws (torch CPU cast).
* up-projection inputs (the expert FFN's first GEMM, whose output is X): with
  hidden = N and I = K, X1 rows N(0,1) float32 from ``SeedSequence([s, 3,
  chunk])`` per 4096-row chunk, [M][hidden]; W1_e = [gate; up] N(0,1)/sqrt(hidden)
  float32 from ``SeedSequence([s, 4, e])``, stored [E_l][2I][hidden]; both bf16.
* fp8: OCP e4m3fn codes with float32 scales, one per (row, 128-wide K block)
  for X and one per (128 N x 128 K block) for W_e: scale = amax/448 (1 when
  amax = 0), code = e4m3fn(v / scale) with round-to-nearest-even, so that
  dequantised value = code * scale.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np
import torch

from .configs import EpConfig

_X_CHUNK = 4096
_FP8_MAX = 448.0


@dataclass
class EpInputs:
    cfg: EpConfig
    topk_ids: np.ndarray        # int32 [R][T][top_k] global expert ids
    topk_w: np.ndarray          # float32 [R][T][top_k] routing weights
    offsets: np.ndarray         # int32 [E_l*R + 1]
    src_info: np.ndarray        # int32 [M][2] = (src_idx t, src_topk k)
    x: np.ndarray               # uint16 bf16 bits [M][K]  or uint8 e4m3fn codes [M][K]
    w: np.ndarray               # uint16 bf16 bits [E_l][N][K] or uint8 codes
    x_scale: np.ndarray | None  # float32 [M][K/128] (fp8 only)
    w_scale: np.ndarray | None  # float32 [E_l][N/128][K/128] (fp8 only)

    @property
    def m_total(self) -> int:
        return int(self.offsets[-1])

    def group_sizes(self) -> np.ndarray:
        R, El = self.cfg.n_ranks, self.cfg.n_experts_local
        b = self.offsets[0::R][: El + 1]
        return np.diff(b.astype(np.int64))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _routing(cfg: EpConfig):
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 0]))
    R, T, Eg, k = cfg.n_ranks, cfg.tokens_per_rank, cfg.n_experts_global, cfg.top_k
    if cfg.routing == "uniform":
        keys = rng.random((R, T, Eg))
    elif cfg.routing == "zipf":
        perm = rng.permutation(Eg)
        logp = -cfg.zipf_s * np.log(perm.astype(np.float64) + 1.0)
        if cfg.n_forced_empty:
            lo = cfg.my_rank * cfg.n_experts_local
            local = np.arange(lo, lo + cfg.n_experts_local)
            coldest = local[np.argsort(logp[local], kind="stable")[: cfg.n_forced_empty]]
            logp[coldest] = -np.inf
        if np.count_nonzero(np.isfinite(logp)) < k:
            raise ValueError("fewer experts with nonzero popularity than top_k")
        u = rng.random((R, T, Eg))
        u = np.clip(u, np.finfo(np.float64).tiny, 1.0)
        keys = logp[None, None, :] - np.log(-np.log(u))
    else:
        raise ValueError(f"unknown routing {cfg.routing!r}")
    part = np.argpartition(-keys, k - 1, axis=-1)[..., :k]
    order = np.argsort(-np.take_along_axis(keys, part, axis=-1), axis=-1, kind="stable")
    ids = np.take_along_axis(part, order, axis=-1).astype(np.int32)
    logits = rng.standard_normal((R, T, k))
    z = np.exp(logits - logits.max(axis=-1, keepdims=True))
    w = (z / z.sum(axis=-1, keepdims=True)).astype(np.float32)
    return ids, w


def _dispatch_layout(cfg: EpConfig, ids: np.ndarray):
    R, T, k, El = cfg.n_ranks, cfg.tokens_per_rank, cfg.top_k, cfg.n_experts_local
    lo = cfg.my_rank * El
    rk, t, kk = np.meshgrid(np.arange(R), np.arange(T), np.arange(k), indexing="ij")
    sel = (ids >= lo) & (ids < lo + El)
    e = (ids[sel] - lo).astype(np.int64)
    rk, t, kk = rk[sel], t[sel], kk[sel]          # already in (rk, t, k) order
    grp = e * R + rk
    order = np.argsort(grp, kind="stable")
    counts = np.bincount(grp, minlength=El * R)
    offsets = np.zeros(El * R + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    src_info = np.stack([t[order], kk[order]], axis=1).astype(np.int32)
    return offsets.astype(np.int32), np.ascontiguousarray(src_info)


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    a = np.clip(a, -_FP8_MAX, _FP8_MAX).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _block_scales(amax: np.ndarray) -> np.ndarray:
    s = (amax / np.float32(_FP8_MAX)).astype(np.float32)
    s[amax == 0] = 1.0
    return s


def _quant_rows(x: np.ndarray):
    """Per (row, 128-wide K block) e4m3fn quantisation of a float32 [M][K]."""
    M, K = x.shape
    xb = x.reshape(M, K // 128, 128)
    scale = _block_scales(np.abs(xb).max(axis=-1))
    q = _to_e4m3_codes(xb / scale[..., None]).reshape(M, K)
    return q, scale


def _quant_blocks(w: np.ndarray):
    """Per (128 N x 128 K block) e4m3fn quantisation of a float32 [N][K]."""
    N, K = w.shape
    wb = w.reshape(N // 128, 128, K // 128, 128)
    scale = _block_scales(np.abs(wb).max(axis=(1, 3)))
    q = _to_e4m3_codes(wb / scale[:, None, :, None]).reshape(N, K)
    return q, scale


def make_routing(cfg: EpConfig):
    """Routing and dispatched-row layout only: (topk_ids, topk_w, offsets, src_info)."""
    ids, tw = _routing(cfg)
    offsets, src_info = _dispatch_layout(cfg, ids)
    return ids, tw, offsets, src_info


def make_inputs(cfg: EpConfig) -> EpInputs:
    """Draw every input of one EP-combine step for ``cfg`` (deterministic in cfg.seed)."""
    R, El, K, N = cfg.n_ranks, cfg.n_experts_local, cfg.k, cfg.n
    if cfg.dtype not in ("bf16", "fp8"):
        raise ValueError(f"unknown dtype {cfg.dtype!r}")
    if cfg.dtype == "fp8" and (K % 128 or N % 128):
        raise ValueError("fp8 block scales need K and N multiples of 128")
    ids, tw, offsets, src_info = make_routing(cfg)
    M = int(offsets[-1])
    fp8 = cfg.dtype == "fp8"

    def x_chunk(c):
        r0, r1 = c * _X_CHUNK, min(M, (c + 1) * _X_CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 1, c]))
        v = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        return _quant_rows(v) if fp8 else (_to_bf16_bits(v), None)

    def w_expert(e):
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 2, e]))
        v = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
        return _quant_blocks(v) if fp8 else (_to_bf16_bits(v), None)

    nchunks = (M + _X_CHUNK - 1) // _X_CHUNK
    with ThreadPoolExecutor(_threads()) as ex:
        xs = list(ex.map(x_chunk, range(nchunks)))
        ws = list(ex.map(w_expert, range(El)))
    xdt = np.uint8 if fp8 else np.uint16
    x = np.concatenate([a for a, _ in xs], axis=0) if xs else np.zeros((0, K), xdt)
    w = np.stack([a for a, _ in ws], axis=0)
    x_scale = w_scale = None
    if fp8:
        x_scale = (np.concatenate([s for _, s in xs], axis=0) if xs
                   else np.zeros((0, K // 128), np.float32))
        w_scale = np.stack([s for _, s in ws], axis=0)
    return EpInputs(cfg, ids, tw, offsets, src_info, np.ascontiguousarray(x),
                    np.ascontiguousarray(w), x_scale, w_scale)


def make_up_inputs(cfg: EpConfig, m_total: int):
    """X1 [M][hidden] and W1 [E_l][2I][hidden] as bf16 codes (uint16) for the
    up-projection of ``cfg`` (hidden = cfg.n, I = cfg.k); M = m_total rows laid
    out in the same grouped order as X."""
    El, I, H = cfg.n_experts_local, cfg.k, cfg.n

    def x_chunk(c):
        r0, r1 = c * _X_CHUNK, min(m_total, (c + 1) * _X_CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 3, c]))
        return _to_bf16_bits(rng.standard_normal((r1 - r0, H), dtype=np.float32))

    def w_expert(e):
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 4, e]))
        v = rng.standard_normal((2 * I, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
        return _to_bf16_bits(v)

    nchunks = (m_total + _X_CHUNK - 1) // _X_CHUNK
    with ThreadPoolExecutor(_threads()) as ex:
        xs = list(ex.map(x_chunk, range(nchunks)))
        ws = list(ex.map(w_expert, range(El)))
    x1 = np.concatenate(xs, axis=0) if xs else np.zeros((0, H), np.uint16)
    return np.ascontiguousarray(x1), np.ascontiguousarray(np.stack(ws, axis=0))

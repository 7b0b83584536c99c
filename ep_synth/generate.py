"""Seeded input generator (numpy + torch CPU casts; no GPU, none of the method's
arithmetic: no locality test, no grouping, no products).

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
* X rows: one row per pick, keyed by the pick itself: the row of pick
  (rk, t, k) is N(0,1) float32 of width K from ``SeedSequence([s, 1, rk, t, k])``.
  The generator knows nothing of which picks are local or how rows are
  grouped: a caller asks for the rows of the picks its own grouping keeps, in
  its own order, and every caller gets the same values for the same pick.
* W_e: N(0,1)/sqrt(K) float32 from ``SeedSequence([s, 2, e])``, stored
  K-contiguous as ``[E_l][N][K]`` (the logical K x N matrix, transposed).
* bf16: round-to-nearest-even cast of the float32 draws (torch CPU cast).
* up-projection inputs (the expert FFN's first GEMM, whose output is X): with
  hidden = N and I = K, the X1 row of pick (rk, t, k) N(0,1) float32 of width
  hidden from ``SeedSequence([s, 3, rk, t, k])``; W1_e = [gate; up] N(0,1)/sqrt(hidden)
  float32 from ``SeedSequence([s, 4, e])``, stored [E_l][2I][hidden]; both bf16.
* token rows (the dispatch's input): rank rk's T rows of width hidden = N,
  N(0,1) float32 from ``SeedSequence([s, 5, rk])``, bf16.
* fp8: OCP e4m3fn codes with float32 scales, one per (row, 128-wide K block)
  for X and one per (128 N x 128 K block) for W_e: scale = amax/448 (1 when
  amax = 0), code = e4m3fn(v / scale) with round-to-nearest-even, so that
  dequantised value = code * scale.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import hashlib
import os

import numpy as np
import torch

from .configs import EpConfig

_FP8_MAX = 448.0


@dataclass
class EpInputs:
    """Routing and weights of one workload; X rows are drawn per pick on demand
    (``rows``), in whatever row order the caller's grouping gives."""
    cfg: EpConfig
    topk_ids: np.ndarray        # int32 [R][T][top_k] global expert ids
    topk_w: np.ndarray          # float32 [R][T][top_k] routing weights
    w: np.ndarray               # uint16 bf16 bits [E_l][N][K] or uint8 e4m3fn codes
    w_scale: np.ndarray | None  # float32 [E_l][N/128][K/128] (fp8 only)
    _last: dict = field(default_factory=dict, repr=False)

    def rows(self, picks):
        """X rows of ``picks`` (int [M][3] of (rk, t, k)), in that order:
        (x [M][K] bf16 bits or e4m3fn codes, x_scale [M][K/128] float32 or None).
        The last answer is kept, so asking again for the same picks costs
        nothing (the arrays returned are then shared: do not modify them)."""
        p = _pick_array(picks)
        key = hashlib.sha1(p.tobytes()).hexdigest()
        if self._last.get("key") != key:
            self._last.clear()
            self._last.update(key=key, value=pick_rows(self.cfg, p))
        return self._last["value"]

    def up_rows(self, picks):
        """Up-projection input rows X1 [M][hidden] of ``picks``: bf16 bits, or
        for fp8 workloads (e4m3fn codes, float32 scales [M][hidden/128])."""
        return pick_up_rows(self.cfg, picks)

    def up_weights(self):
        """Up-projection weights W1 [E_l][2I][hidden]: bf16 bits, or for fp8
        workloads (e4m3fn codes, float32 scales [E_l][2I/128][hidden/128])."""
        return make_up_weights(self.cfg)

    def tokens(self):
        """Token hidden rows of every source rank, [R][T][hidden]: bf16 bits,
        or for fp8 workloads (e4m3fn codes, float32 scales [R][T][hidden/128])."""
        return make_tokens(self.cfg)


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
    """Routing only: (topk_ids int32 [R][T][top_k], topk_w float32 [R][T][top_k])."""
    return _routing(cfg)


def _pick_array(picks) -> np.ndarray:
    p = np.asarray(picks, dtype=np.int64).reshape(-1, 3)
    return p


def _row_stream(cfg: EpConfig, stream: int, pick, width: int) -> np.ndarray:
    rk, t, k = (int(v) for v in pick)
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, stream, rk, t, k]))
    return rng.standard_normal(width, dtype=np.float32)


def pick_rows(cfg: EpConfig, picks):
    """X rows of the given picks, one N(0,1) float32 row of width K per pick
    (rk, t, k) from ``SeedSequence([seed, 1, rk, t, k])``, as bf16 bits or, for
    fp8 workloads, e4m3fn codes with their per-128 block scales.  The value of
    a pick's row does not depend on which other picks are asked for or in
    which order."""
    p = _pick_array(picks)
    M, K = p.shape[0], cfg.k
    fp8 = cfg.dtype == "fp8"
    if fp8 and K % 128:
        raise ValueError("fp8 block scales need K a multiple of 128")
    v = np.empty((M, K), dtype=np.float32)
    for i in range(M):
        v[i] = _row_stream(cfg, 1, p[i], K)
    if fp8:
        if M == 0:
            return np.zeros((0, K), np.uint8), np.zeros((0, K // 128), np.float32)
        q, s = _quant_rows(v)
        return np.ascontiguousarray(q), np.ascontiguousarray(s)
    return _to_bf16_bits(v), None


def make_weights(cfg: EpConfig):
    """W_e of every local expert: (w [E_l][N][K] bf16 bits or e4m3fn codes,
    w_scale [E_l][N/128][K/128] float32 or None)."""
    El, K, N = cfg.n_experts_local, cfg.k, cfg.n
    fp8 = cfg.dtype == "fp8"
    if fp8 and (K % 128 or N % 128):
        raise ValueError("fp8 block scales need K and N multiples of 128")

    def w_expert(e):
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 2, e]))
        v = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
        return _quant_blocks(v) if fp8 else (_to_bf16_bits(v), None)

    with ThreadPoolExecutor(_threads()) as ex:
        ws = list(ex.map(w_expert, range(El)))
    w = np.ascontiguousarray(np.stack([a for a, _ in ws], axis=0))
    w_scale = np.ascontiguousarray(np.stack([s for _, s in ws], axis=0)) if fp8 else None
    return w, w_scale


def make_inputs(cfg: EpConfig) -> EpInputs:
    """Draw the routing and weights of one EP-combine step for ``cfg``
    (deterministic in cfg.seed); X rows come per pick from ``EpInputs.rows``."""
    if cfg.dtype not in ("bf16", "fp8"):
        raise ValueError(f"unknown dtype {cfg.dtype!r}")
    ids, tw = make_routing(cfg)
    w, w_scale = make_weights(cfg)
    return EpInputs(cfg, ids, tw, w, w_scale)


def pick_up_rows(cfg: EpConfig, picks):
    """Up-projection input rows X1 (hidden = cfg.n wide) of the given picks,
    N(0,1) from ``SeedSequence([seed, 3, rk, t, k])``: bf16 bits, or for fp8
    workloads e4m3fn codes with their per (row, 128 block) scales."""
    p = _pick_array(picks)
    v = np.empty((p.shape[0], cfg.n), dtype=np.float32)
    for i in range(p.shape[0]):
        v[i] = _row_stream(cfg, 3, p[i], cfg.n)
    return _quant_rows(v) if cfg.dtype == "fp8" else _to_bf16_bits(v)


def make_tokens(cfg: EpConfig):
    """Hidden rows of every token of every source rank, [R][T][hidden] bf16
    bits with hidden = cfg.n: N(0,1) from ``SeedSequence([seed, 5, rk])`` per
    rank.  The input of the dispatch (each local pick's row is its token's)."""
    fp8 = cfg.dtype == "fp8"

    def rank_rows(rk):
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 5, rk]))
        v = rng.standard_normal((cfg.tokens_per_rank, cfg.n), dtype=np.float32)
        return _quant_rows(v) if fp8 else (_to_bf16_bits(v), None)

    with ThreadPoolExecutor(_threads()) as ex:
        rows = list(ex.map(rank_rows, range(cfg.n_ranks)))
    codes = np.ascontiguousarray(np.stack([r for r, _ in rows], axis=0))
    if not fp8:
        return codes
    return codes, np.ascontiguousarray(np.stack([s for _, s in rows], axis=0))


def make_up_weights(cfg: EpConfig):
    """W1 [E_l][2I][hidden] bf16 bits for the up-projection of ``cfg``
    (hidden = cfg.n, I = cfg.k): gate rows 0..I-1, then up rows."""
    El, I, H = cfg.n_experts_local, cfg.k, cfg.n

    fp8 = cfg.dtype == "fp8"

    def w_expert(e):
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, 4, e]))
        v = rng.standard_normal((2 * I, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
        return _quant_blocks(v) if fp8 else (_to_bf16_bits(v), None)

    with ThreadPoolExecutor(_threads()) as ex:
        ws = list(ex.map(w_expert, range(El)))
    codes = np.ascontiguousarray(np.stack([w for w, _ in ws], axis=0))
    if not fp8:
        return codes
    return codes, np.ascontiguousarray(np.stack([s for _, s in ws], axis=0))

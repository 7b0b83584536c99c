"""Plain CPU oracle for the MoE expert-parallel combine (grouped GEMM + row scatter
+ completion signalling + top-k weighted combine).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package entry
module and the ``cpu_baseline`` leg of the benchmark may import this package.
The HIP library never calls it, and this package imports nothing from the HIP
path: the two share no code, only the seeded inputs drawn by ``ep_synth``.

Everything here is the plain definition written out, with library primitives (a
matrix product, a sort) used only as whole steps.  The values the parity tests
compare with are computed as the method states them: the expert GEMM with
binary32 products and binary32 accumulation (a float32 matrix product), the
combine with one binary32 fused multiply-add per pick in ascending pick order
(``combine.c``, built by ``_build_clib``), each result rounded once to bf16.
The same GEMM in float64 (``*_f64``), an exact sum up to float64 rounding, is
kept as the reference the binary32 forms are pinned against.  The passages each
function follows are cited by page title and section:

* "EpiloguePeerSink" (Mojo trait page), description and ``send_tile`` args:
  a finished output tile goes straight to the ranks owning its rows instead of
  a local C; rows past ``m_end`` (exclusive bound of the tile's group) are not
  part of the group; ``expert_id`` is the logical per-rank expert slot.
* "P3PeerSendConfig" (Mojo struct page), description: the count word of
  (expert e, rank rk) sits at linear index ``e*n_ranks + rk``; the receive-buffer
  slot of (src_idx, src_topk, byte_off) sits at byte
  ``(src_idx*top_k + src_topk)*msg_bytes + byte_off``; receive offsets are bounds
  checked; fields ``recv_buf_ptrs`` (one buffer per rank, at most 8),
  ``max_tokens_per_rank``, ``top_k``, ``msg_bytes``.  The blockwise fp8 kernel
  family named there has 1-D activation and 2-D weight scales.
* "ep_signal_completion" (Mojo function page), description and parameters:
  with rank-level completion each expert's count word is a plain progress store
  made before an acquire-release election on the destination rank's counter;
  the producer elected last (after ``n_experts_per_device`` signals) release-
  stores the rank-completion flag kept in the tail of the count buffer; the
  consumer acquires that flag once per source rank.

Readings of what the pages leave open (each is listed in the design notes):
row layout of the grouped input, bf16 rounding of the stored row and of the
combined output, the published signal being the row count, the flag value
being the step's epoch, combine over the local picks only (+0 for a token with
none), and fp8 = OCP e4m3fn with 1x128 / 128x128 float32 scales.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16", "e4m3fn_to_f64", "bf16_to_f32", "e4m3fn_to_f32",
    "recv_count_index", "recv_slot_offset",
    "group_local_picks", "row_owner", "row_picks", "dispatch_rows",
    "f32_to_e4m3fn", "quantize_rows_e4m3",
    "expert_rows_bf16", "expert_rows_fp8", "expert_swiglu", "expert_swiglu_fp8",
    "expert_rows_bf16_f64", "expert_rows_fp8_f64", "expert_swiglu_f64",
    "scatter_rows", "recv_counts", "final_control", "ElectionModel",
    "combine_tokens", "combine_picks_fmaf", "run_step", "ORACLE_ERR_SLOT_OOB",
]

ORACLE_ERR_SLOT_OOB = 1


# ---------------------------------------------------------------- number formats

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 code -> value.  A bf16 code is the upper 16 bits of an IEEE binary32,
    so widening is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 code, rounding once to nearest, ties to even.

    bf16 keeps 8 significant bits and binary32's exponent range (normal binades
    2^-126 .. 2^127, subnormal spacing 2^-133).  The value is rounded directly
    from float64 (no intermediate binary32 rounding): q = rint(|x| / ulp), where
    ulp is the spacing of the binade holding |x|; magnitudes that round past the
    largest finite value become infinity.  NaN maps to the quiet NaN 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(ax)                      # ax = m * 2^ex with 0.5 <= m < 1
    binade = np.maximum(ex.astype(np.int64) - 1, -126)
    ulp = np.ldexp(1.0, (binade - 7).astype(np.int64))
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(ax / ulp) * ulp           # exact: scaling by a power of two
        f32 = r.astype(np.float32)            # exact unless it overflows to inf
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def e4m3fn_to_f64(codes) -> np.ndarray:
    """OCP fp8 e4m3fn code -> value: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; codes
    0x7F / 0xFF are NaN; there is no infinity (largest finite is 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = (c & 7).astype(np.float64)
    mag = np.where(ef == 0, mf / 8.0 * 2.0 ** -6,
                   (1.0 + mf / 8.0) * np.ldexp(1.0, (ef - 7)))
    val = sign * mag
    return np.where((ef == 15) & ((c & 7) == 7), np.nan, val)


def f32_to_e4m3fn(values) -> np.ndarray:
    """binary32 value -> OCP e4m3fn code, rounded to nearest with ties to the
    even code.  From the format (see ``e4m3fn_to_f64``): a magnitude below
    2^-6 is k * 2^-9 with k = 0..7 in the subnormal codes (k = 8 is the
    smallest normal, code 8); above it a = 2^e * (1 + m/8), code
    (e + 7) << 3 | m.  Magnitudes that would round past 448 (the largest
    finite value) give 448.  Written with ``frexp`` so that no rounding of its
    own enters: every intermediate is exact in float64."""
    v = np.asarray(values, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    frac, exp2 = np.frexp(a)                      # a = frac * 2^exp2, frac in [0.5, 1)
    e = exp2.astype(np.int64) - 1                 # a = 2^e * (2 frac), 2 frac in [1, 2)
    normal = a >= 2.0 ** -6
    # normal: mantissa steps of 1/8 of the binade, RNE; a carry moves to the next binade
    m = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code_n = np.minimum(((e + 7) << 3) | m, 0x7E)
    # subnormal: steps of 2^-9, RNE (k = 8 is code 8, the smallest normal)
    code_s = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    return (sign | code).astype(np.uint8)


def quantize_rows_e4m3(h):
    """Per (row, 128-wide block) e4m3fn quantisation, the 1-D activation
    scaling of the blockwise fp8 family ("P3PeerSendConfig", description), in
    binary32: scale = amax / 448 (1 for a block of zeros), code = RNE(h / scale).
    h: float32 [M][I], I a multiple of 128.  Returns (codes uint8 [M][I],
    scales float32 [M][I/128])."""
    h = np.asarray(h, dtype=np.float32)
    M, I = h.shape
    hb = h.reshape(M, I // 128, 128)
    amax = np.abs(hb).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    v = (hb / scale[..., None]).astype(np.float32)
    return f32_to_e4m3fn(v).reshape(M, I), scale


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 code -> binary32 value (exact: the code is a binary32's upper half)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def e4m3fn_to_f32(codes) -> np.ndarray:
    """e4m3fn code -> binary32 value (exact: every e4m3fn value is a binary32)."""
    return e4m3fn_to_f64(codes).astype(np.float32)


# ---------------------------------------------------------------- index formulas
# "P3PeerSendConfig", description: the two row-major linear-index formulas.

def recv_count_index(e, rk, n_ranks):
    """Linear index of the count word for (local expert e, rank rk)."""
    return e * n_ranks + rk


def recv_slot_offset(src_idx, src_topk, byte_off, top_k, msg_bytes):
    """Byte offset, in its owner's receive buffer, of byte ``byte_off`` of the
    message for pick ``src_topk`` of token ``src_idx``."""
    return (src_idx * top_k + src_topk) * msg_bytes + byte_off


# ---------------------------------------------------------------- routing -> groups

def group_local_picks(topk_ids, n_experts_per_device, my_rank):
    """Rows this GPU computes, in grouped order.

    A pick (rk, t, k) with global expert g is local when g lies in
    [my_rank*E_l, (my_rank+1)*E_l); its local expert slot is e = g - my_rank*E_l
    ("EpiloguePeerSink", ``send_tile`` arg ``expert_id``).  Rows are sorted by
    (e, rk, t, k); group e is the row range [offsets[e*R], offsets[(e+1)*R]) and
    offsets[e*R + rk] starts the run of rank rk inside it (reading of the
    dispatch layout).  Returns (offsets int64 [E_l*R+1], src_info int64 [M][2]
    holding (t, k) per row)."""
    ids = np.asarray(topk_ids)
    R, T, K = ids.shape
    El = n_experts_per_device
    lo = my_rank * El
    rk, t, k = np.meshgrid(np.arange(R), np.arange(T), np.arange(K), indexing="ij")
    g = ids.astype(np.int64)
    local = (g >= lo) & (g < lo + El)
    e, rk, t, k = g[local] - lo, rk[local], t[local], k[local]
    order = np.lexsort((k, t, rk, e))         # last key is the primary key
    e, rk, t, k = e[order], rk[order], t[order], k[order]
    offsets = np.zeros(El * R + 1, dtype=np.int64)
    for gi in range(El * R):                  # run boundaries of every (e, rk)
        offsets[gi + 1] = offsets[gi] + np.count_nonzero(e * R + rk == gi)
    return offsets, np.stack([t, k], axis=1).astype(np.int64)


def row_owner(offsets, n_ranks, m):
    """(local expert e, source rank rk) of grouped row m."""
    gi = int(np.searchsorted(np.asarray(offsets), m, side="right")) - 1
    return gi // n_ranks, gi % n_ranks


def row_picks(offsets, src_info, n_ranks):
    """The pick (rk, t, k) of every grouped row, int64 [M][3]: the owner rank
    from the run the row falls in, (t, k) from src_info.  The rows' inputs are
    drawn per pick, so this is how a grouping asks for its rows."""
    off = np.asarray(offsets, dtype=np.int64)
    M = int(off[-1])
    gi = np.searchsorted(off, np.arange(M), side="right") - 1
    src = np.asarray(src_info, dtype=np.int64).reshape(-1, 2)[:M]
    return np.stack([gi % n_ranks, src[:, 0], src[:, 1]], axis=1).astype(np.int64)


def dispatch_rows(token_rows, offsets, src_info, n_ranks):
    """Input rows of the expert FFN on this GPU's share: grouped row m gets the
    row of its pick's token, token_rows[rk][t] (every local pick of a token
    gets the same row).  The sink of "P3PeerSendConfig" (description) sits in
    the FFN's second GEMM; this is what its first GEMM reads.  ``token_rows``
    is [R][T][...]; returns [M][...]."""
    picks = row_picks(offsets, src_info, n_ranks)
    tr = np.asarray(token_rows)
    return tr[picks[:, 0], picks[:, 1]] if picks.shape[0] else tr.reshape(-1, *tr.shape[2:])[:0]


def _group_bounds(offsets, n_ranks, e):
    return int(offsets[e * n_ranks]), int(offsets[(e + 1) * n_ranks])


# ---------------------------------------------------------------- expert GEMM

def _rows_of_group(rows, offsets, n_ranks, e):
    lo, hi = _group_bounds(offsets, n_ranks, e)
    return np.nonzero((rows >= lo) & (rows < hi))[0]


def expert_rows_bf16(x_bits, w_bits, offsets, n_ranks, rows=None):
    """The expert GEMM as computed on the path: y[m][n] = sum_k X[m][k] *
    W_e[k][n] for each requested row m of group e ("EpiloguePeerSink",
    send_tile: the tile of expert ``expert_id`` over rows before ``m_end``), with
    binary32 products (exact for bf16 operands) and binary32 accumulation, the
    float32 matrix product of the decoded codes; the order of the sum is the
    library's.  ``w_bits`` stores the logical K x N matrix W_e K-contiguous, as
    [E_l][N][K].  Returns float32 [len(rows)][N] (before rounding)."""
    x_bits = np.asarray(x_bits)
    w_bits = np.asarray(w_bits)
    El = w_bits.shape[0]
    rows = np.arange(x_bits.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((rows.size, w_bits.shape[1]), dtype=np.float32)
    for e in range(El):
        sel = _rows_of_group(rows, offsets, n_ranks, e)
        if sel.size == 0:
            continue
        xe = bf16_to_f32(x_bits[rows[sel]])
        we = bf16_to_f32(w_bits[e])           # [N][K]
        y[sel] = xe @ we.T
    return y


def expert_rows_fp8(xq, x_scale, wq, w_scale, offsets, n_ranks, rows=None):
    """Blockwise-scaled fp8 product in binary32 ("P3PeerSendConfig", description:
    the blockwise fp8 family with 1-D activation and 2-D weight scales):
    y[m][n] = sum_b (x_scale[m][b] * w_scale[e][n//128][b])
                    * (sum_{k in block b} X[m][k] * W_e[k][n]),
    each block's sum a float32 matrix product of the decoded codes, scaled and
    added into the binary32 result block by block in ascending b.  Returns
    float32 [len(rows)][N]."""
    xq = np.asarray(xq)
    wq = np.asarray(wq)
    El, N, K = wq.shape
    rows = np.arange(xq.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((rows.size, N), dtype=np.float32)
    for e in range(El):
        sel = _rows_of_group(rows, offsets, n_ranks, e)
        if sel.size == 0:
            continue
        xe = e4m3fn_to_f32(xq[rows[sel]])     # [r][K]
        we = e4m3fn_to_f32(wq[e])             # [N][K]
        sx = np.asarray(x_scale, dtype=np.float32)[rows[sel]]              # [r][nb]
        sw = np.repeat(np.asarray(w_scale, dtype=np.float32)[e], 128, axis=0)  # [N][nb]
        acc = np.zeros((sel.size, N), dtype=np.float32)
        for b in range(K // 128):
            ks = slice(b * 128, (b + 1) * 128)
            part = xe[:, ks] @ we[:, ks].T
            acc += part * (sx[:, b:b + 1] * sw[:, b][None, :])
        y[sel] = acc
    return y


def expert_rows_bf16_f64(x_bits, w_bits, offsets, n_ranks, rows=None):
    """Reference form of ``expert_rows_bf16``: the same sum in float64 (exact
    products, one float64 rounding per addition), against which the binary32
    result is pinned.  Returns float64 [len(rows)][N] (before rounding)."""
    x_bits = np.asarray(x_bits)
    w_bits = np.asarray(w_bits)
    El = w_bits.shape[0]
    M = x_bits.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((rows.size, w_bits.shape[1]), dtype=np.float64)
    for e in range(El):
        lo, hi = _group_bounds(offsets, n_ranks, e)
        sel = np.nonzero((rows >= lo) & (rows < hi))[0]
        if sel.size == 0:
            continue
        xe = bf16_to_f64(x_bits[rows[sel]])
        we = bf16_to_f64(w_bits[e])           # [N][K]
        y[sel] = xe @ we.T
    return y


def expert_rows_fp8_f64(xq, x_scale, wq, w_scale, offsets, n_ranks, rows=None):
    """Reference form of ``expert_rows_fp8`` in float64:
    y[m][n] = sum_b x_scale[m][b] * w_scale[e][n//128][b]
                    * sum_{k in block b} X[m][k] * W_e[k][n],
    with X, W_e the decoded e4m3fn codes and b running over 128-wide K blocks.
    Returns float64 [len(rows)][N]."""
    xq = np.asarray(xq)
    wq = np.asarray(wq)
    El, N, K = wq.shape
    nb = K // 128
    M = xq.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((rows.size, N), dtype=np.float64)
    for e in range(El):
        lo, hi = _group_bounds(offsets, n_ranks, e)
        sel = np.nonzero((rows >= lo) & (rows < hi))[0]
        if sel.size == 0:
            continue
        xe = e4m3fn_to_f64(xq[rows[sel]])     # [r][K]
        we = e4m3fn_to_f64(wq[e])             # [N][K]
        sx = np.asarray(x_scale, dtype=np.float64)[rows[sel]]            # [r][nb]
        sw = np.repeat(np.asarray(w_scale, dtype=np.float64)[e], 128, axis=0)  # [N][nb]
        for b in range(nb):
            ks = slice(b * 128, (b + 1) * 128)
            part = xe[:, ks] @ we[:, ks].T
            y[sel] += part * sx[:, b:b + 1] * sw[:, b][None, :]
    return y


# ---------------------------------------------------------------- up-projection

def expert_swiglu(x1_bits, w1_bits, offsets, n_ranks, rows=None):
    """The expert FFN's first GEMM with SwiGLU, whose output is X of the
    down-projection (the sink of "EpiloguePeerSink" / "P3PeerSendConfig" sits in
    the epilogue of the FFN's second GEMM, so a first one feeds it).  For row m
    of group e, with W1_e = [gate; up] stored [2I][hidden]:
        g = sum_k X1[m][k] * W1_e[i][k],  u = sum_k X1[m][k] * W1_e[I + i][k],
        h[m][i] = silu(g) * u,  silu(g) = g / (1 + exp(-g)),
    sums as in ``expert_rows_bf16`` and the activation in binary32.  Returns
    float32 [len(rows)][I] (before rounding)."""
    gu = expert_rows_bf16(x1_bits, w1_bits, offsets, n_ranks, rows)
    half = gu.shape[1] // 2
    g, u = gu[:, :half], gu[:, half:]
    with np.errstate(over="ignore"):
        return g / (np.float32(1) + np.exp(-g)) * u


def expert_swiglu_fp8(x1q, x1_scale, w1q, w1_scale, offsets, n_ranks, rows=None):
    """``expert_swiglu`` on block-scaled fp8 operands: gate and up sums as in
    ``expert_rows_fp8`` (W1_e = [gate; up] stored [2I][hidden] with w1_scale
    [2I/128][hidden/128]), the activation in binary32.  Returns float32
    [len(rows)][I] (before ``quantize_rows_e4m3``)."""
    gu = expert_rows_fp8(x1q, x1_scale, w1q, w1_scale, offsets, n_ranks, rows)
    half = gu.shape[1] // 2
    g, u = gu[:, :half], gu[:, half:]
    with np.errstate(over="ignore"):
        return g / (np.float32(1) + np.exp(-g)) * u


def expert_swiglu_f64(x1_bits, w1_bits, offsets, n_ranks, rows=None):
    """Reference form of ``expert_swiglu``, all in float64.  Returns float64
    [len(rows)][I] (before rounding)."""
    gu = expert_rows_bf16_f64(x1_bits, w1_bits, offsets, n_ranks, rows)
    half = gu.shape[1] // 2
    g, u = gu[:, :half], gu[:, half:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


# ---------------------------------------------------------------- scatter + counts

def scatter_rows(y_bits, rows, offsets, src_info, recv_bufs, *, n_ranks, top_k,
                 msg_bytes, max_tokens_per_rank):
    """Write each row's bf16 message into its owner's receive buffer
    ("EpiloguePeerSink": the tile goes to the peers owning the rows;
    "P3PeerSendConfig": slot formula and receive-offset bounds check).

    ``y_bits`` is uint16 [len(rows)][N]; ``recv_bufs`` is a list of R uint8
    arrays.  The message occupies bytes [0, 2N) of its slot; bytes [2N,
    msg_bytes) are not touched.  A slot whose token index or pick index is out
    of range, or whose message would end past the buffer, is not written and
    the error bit ORACLE_ERR_SLOT_OOB is returned."""
    err = 0
    cap = max_tokens_per_rank * top_k * msg_bytes
    for i, m in enumerate(np.asarray(rows, dtype=np.int64)):
        _, rk = row_owner(offsets, n_ranks, m)
        t, k = int(src_info[m][0]), int(src_info[m][1])
        msg = np.ascontiguousarray(y_bits[i], dtype="<u2").view(np.uint8)
        off = recv_slot_offset(t, k, 0, top_k, msg_bytes)
        if not (0 <= t < max_tokens_per_rank and 0 <= k < top_k and
                off + msg.size <= cap and msg.size <= msg_bytes):
            err |= ORACLE_ERR_SLOT_OOB
            continue
        recv_bufs[rk][off:off + msg.size] = msg
    return err


def recv_counts(offsets, n_ranks, n_experts_per_device):
    """Count word of every (e, rk): the number of rows of expert e owned by
    rank rk, zero included ("ep_signal_completion", argument signal: the word
    each expert publishes for a rank; reading: the row count)."""
    words = np.zeros(n_experts_per_device * n_ranks, dtype=np.uint64)
    for e in range(n_experts_per_device):
        for rk in range(n_ranks):
            words[recv_count_index(e, rk, n_ranks)] = \
                offsets[e * n_ranks + rk + 1] - offsets[e * n_ranks + rk]
    return words


def final_control(offsets, n_ranks, n_experts_per_device, epoch):
    """Control state after one completed step: E_l*R count words followed by
    R rank-completion flags (the count buffer's tail, "ep_signal_completion",
    parameter has_rank_flag) that all hold ``epoch``; election counters and
    per-expert tile counters are back at zero."""
    words = np.concatenate([recv_counts(offsets, n_ranks, n_experts_per_device),
                            np.full(n_ranks, epoch, dtype=np.uint64)])
    return {"words": words,
            "rank_counter": np.zeros(n_ranks, dtype=np.int64),
            "tile_counter": np.zeros(n_experts_per_device, dtype=np.int64)}


def tagged_count(rows, epoch):
    """Count word of per-expert completion ("ep_signal_completion",
    description: the form without rank-level completion, where a consumer
    looks at the signal of every expert).  Reading: a word is ready when it carries
    the step, so it holds the low 32 bits of the epoch in its high half and the
    row count in its low half."""
    return ((int(epoch) & 0xFFFFFFFF) << 32) | (int(rows) & 0xFFFFFFFF)


def final_control_per_expert(offsets, n_ranks, n_experts_per_device, epoch):
    """Control state after one completed step with per-expert completion, from
    a zeroed control block: every count word tagged with the step, the rank
    flags, election counters and tile counters untouched (zero)."""
    counts = recv_counts(offsets, n_ranks, n_experts_per_device)
    words = np.array([tagged_count(c, epoch) for c in counts] + [0] * n_ranks, dtype=np.uint64)
    return {"words": words,
            "rank_counter": np.zeros(n_ranks, dtype=np.int64),
            "tile_counter": np.zeros(n_experts_per_device, dtype=np.int64)}


class ElectionModel:
    """Sequential model of rank-level completion ("ep_signal_completion",
    description).  A signal for (expert e, destination rank rk) stores the count
    word, then does an atomic fetch-add on rk's election counter; the producer
    that sees the counter at n_experts_per_device - 1 is elected, re-arms the
    counter and stores the rank flag.  Every signal is applied atomically in the
    order given, which is one legal total order of the counter's
    modification order."""

    def __init__(self, n_ranks, n_experts_per_device, epoch):
        self.R, self.El, self.epoch = n_ranks, n_experts_per_device, epoch
        self.words = np.zeros(n_experts_per_device * n_ranks + n_ranks, dtype=np.uint64)
        self.counter = np.zeros(n_ranks, dtype=np.int64)

    def signal(self, e, rk, value) -> bool:
        self.words[recv_count_index(e, rk, self.R)] = value
        old = self.counter[rk]
        self.counter[rk] = old + 1
        if old == self.El - 1:
            self.counter[rk] = 0
            self.words[self.El * self.R + rk] = self.epoch
            return True
        return False

    def flag(self, rk):
        return int(self.words[self.El * self.R + rk])


# ---------------------------------------------------------------- combine

_HERE = os.path.dirname(os.path.abspath(__file__))
_CLIB_SRC = os.path.join(_HERE, "combine.c")
_CLIB = os.path.join(_HERE, "liboracle_combine.so")
_clib_handle = None
_clib_lock = threading.Lock()


def _build_clib(force=False):
    """Compiles combine.c with the host C compiler (plain C, no fast-math
    contractions or reassociation) into liboracle_combine.so next to it, when
    it is missing, older than its source, or ``force``."""
    if (not force and os.path.exists(_CLIB)
            and os.path.getmtime(_CLIB) >= os.path.getmtime(_CLIB_SRC)):
        return _CLIB
    tmp = f"{_CLIB}.{os.getpid()}.tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", _CLIB_SRC, "-o", tmp, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the oracle's combine failed:\n{r.stderr}")
    os.replace(tmp, _CLIB)
    return _CLIB


def _clib():
    global _clib_handle
    with _clib_lock:
        if _clib_handle is None:
            lib = ctypes.CDLL(_build_clib())
            f = lib.oracle_combine_fmaf
            f.restype = None
            f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                          ctypes.c_int64, ctypes.c_void_p]
            _clib_handle = lib
        return _clib_handle


def combine_picks_fmaf(slots, weights, first, n):
    """acc = +0, then acc = fmaf(weight, slot value, acc) over the picks
    [first[i], first[i+1]) of token i in the given order, per column, in
    binary32 (``combine.c``).  ``slots`` uint16 bf16 codes [P][n], ``weights``
    float32 [P], ``first`` int64 [n_tokens + 1].  Returns float32 [n_tokens][n]."""
    slots = np.ascontiguousarray(slots, dtype=np.uint16).reshape(-1, n)
    weights = np.ascontiguousarray(weights, dtype=np.float32).reshape(-1)
    first = np.ascontiguousarray(first, dtype=np.int64).reshape(-1)
    nt = first.size - 1
    if slots.shape[0] != weights.size or int(first[-1]) != weights.size or first[0] != 0:
        raise ValueError("slots, weights and first disagree")
    out = np.empty((nt, n), dtype=np.float32)
    if nt and n:
        _clib().oracle_combine_fmaf(slots.ctypes.data, weights.ctypes.data, first.ctypes.data,
                                    nt, n, out.ctypes.data)
    return out


def combine_tokens(topk_ids, topk_w, recv_bufs, *, n_experts_per_device, my_rank,
                   top_k, msg_bytes, n, as_f32=False):
    """Top-k routing-weighted combine of the slots this GPU's experts wrote
    ("P3PeerSendConfig", description: the combine kernel reads slot (t, k) of
    rank rk; "ep_signal_completion", description: the consumer reads a rank's
    slots once the rank is complete).

    out[rk][t][:] = bf16( acc ),  acc = +0 then, for k = 0..top_k-1 in ascending
    order whose expert is local, acc = fmaf(topk_w[rk][t][k], slot(rk, t, k)[:], acc)
    in binary32; a token with no local pick gets +0.  ``topk_ids`` is
    [R][T][top_k] with T <= the receive buffers' token capacity.  Returns uint16
    bf16 codes [R][T][n] (or the binary32 sums with ``as_f32``)."""
    ids = np.asarray(topk_ids)
    R, T, _ = ids.shape
    lo = my_rank * n_experts_per_device
    out = np.zeros((R, T, n), dtype=np.float32)
    for rk in range(R):
        g = ids[rk].astype(np.int64)
        local = (g >= lo) & (g < lo + n_experts_per_device)
        t_idx, k_idx = np.nonzero(local)          # row-major: t, then k ascending
        first = np.zeros(T + 1, dtype=np.int64)
        np.cumsum(np.count_nonzero(local, axis=1), out=first[1:])
        buf = np.asarray(recv_bufs[rk])[: T * top_k * msg_bytes].reshape(T * top_k, msg_bytes)
        slots = buf[t_idx * top_k + k_idx, : 2 * n].copy().view("<u2")
        weights = np.asarray(topk_w, dtype=np.float32)[rk][t_idx, k_idx]
        out[rk] = combine_picks_fmaf(slots, weights, first, n)
    return out if as_f32 else f64_to_bf16(out.astype(np.float64))


# ---------------------------------------------------------------- whole step

def run_step(*, topk_ids, topk_w, w, n_ranks, n_experts_per_device, top_k,
             msg_bytes, max_tokens_per_rank, my_rank=0, dtype="bf16", x=None,
             x_scale=None, x_rows=None, w_scale=None, epoch=1, sentinel=0xFF,
             per_expert=False):
    """One EP-combine step on this GPU's share, from routing to combined output.

    The grouped row layout is derived here from ``topk_ids``.  The expert input
    rows are either ``x`` ([M][K], already in this grouping's order, with
    ``x_scale`` for fp8) or asked for by pick: ``x_rows(picks)`` returns
    (x, x_scale) for the int [M][3] (rk, t, k) picks of this grouping's rows.
    Receive buffers start filled with ``sentinel`` bytes.  Returns a dict with
    the grouping, the expert outputs (binary32, before rounding) and their bf16
    codes, the receive buffers, the control state, the combined output (uint16
    bf16 codes [R][T][N]) and the error bits."""
    offsets, src_info = group_local_picks(topk_ids, n_experts_per_device, my_rank)
    M = int(offsets[-1])
    if x is None:
        x, x_scale = x_rows(row_picks(offsets, src_info, n_ranks))
    if x.shape[0] != M:
        raise ValueError(f"x has {x.shape[0]} rows, routing gives {M}")
    if dtype == "bf16":
        y = expert_rows_bf16(x, w, offsets, n_ranks)
    elif dtype == "fp8":
        y = expert_rows_fp8(x, x_scale, w, w_scale, offsets, n_ranks)
    else:
        raise ValueError(dtype)
    y_bits = f64_to_bf16(y.astype(np.float64))
    n = y.shape[1]
    cap = max_tokens_per_rank * top_k * msg_bytes
    recv = [np.full(cap, sentinel, dtype=np.uint8) for _ in range(n_ranks)]
    err = scatter_rows(y_bits, np.arange(M), offsets, src_info, recv,
                       n_ranks=n_ranks, top_k=top_k, msg_bytes=msg_bytes,
                       max_tokens_per_rank=max_tokens_per_rank)
    ctrl = (final_control_per_expert if per_expert else final_control)(
        offsets, n_ranks, n_experts_per_device, epoch)
    out = combine_tokens(topk_ids, topk_w, recv, n_experts_per_device=n_experts_per_device,
                         my_rank=my_rank, top_k=top_k, msg_bytes=msg_bytes, n=n)
    return {"topk_ids": np.asarray(topk_ids), "offsets": offsets, "src_info": src_info,
            "x": x, "x_scale": x_scale, "y": y,
            "y_bits": y_bits, "recv_bufs": recv, "control": ctrl, "out_bits": out, "err": err}

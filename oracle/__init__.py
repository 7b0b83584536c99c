"""Plain CPU oracle for the MoE expert-parallel combine (grouped GEMM + row scatter
+ completion signalling + top-k weighted combine).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package entry
module and the ``cpu_baseline`` leg of the benchmark may import this package.
The HIP library never calls it, and this package imports nothing from the HIP
path: the two share no code, only the seeded inputs drawn by ``ep_synth``.

Everything here is the plain definition written out, in float64 with exact
products, and library primitives (a matrix product, a sort) used only as whole
steps.  The passages each function follows are cited by page title and section:

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

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16", "e4m3fn_to_f64",
    "recv_count_index", "recv_slot_offset",
    "group_local_picks", "row_owner",
    "expert_rows_bf16_f64", "expert_rows_fp8_f64", "expert_swiglu_f64",
    "scatter_rows", "recv_counts", "final_control", "ElectionModel",
    "combine_tokens", "sampled_step", "run_step", "ORACLE_ERR_SLOT_OOB",
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


def _group_bounds(offsets, n_ranks, e):
    return int(offsets[e * n_ranks]), int(offsets[(e + 1) * n_ranks])


# ---------------------------------------------------------------- expert GEMM

def expert_rows_bf16_f64(x_bits, w_bits, offsets, n_ranks, rows=None):
    """y[m][n] = sum_k X[m][k] * W_e[k][n] in float64, for each requested row m
    of group e.  ``w_bits`` stores the logical K x N matrix W_e K-contiguous,
    as [E_l][N][K].  Returns float64 [len(rows)][N] (before rounding)."""
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
    """Blockwise-scaled fp8 product ("P3PeerSendConfig", description: the
    blockwise_fp8_1d2d family, 1-D activation / 2-D weight scales):
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

def expert_swiglu_f64(x1_bits, w1_bits, offsets, n_ranks, rows=None):
    """The expert FFN's first GEMM with SwiGLU, whose output is X of the
    down-projection (the sink of "EpiloguePeerSink" / "P3PeerSendConfig" sits in
    the epilogue of the FFN's second GEMM, so a first one feeds it).  For row m
    of group e, with W1_e = [gate; up] stored [2I][hidden]:
        g = sum_k X1[m][k] * W1_e[i][k],  u = sum_k X1[m][k] * W1_e[I + i][k],
        h[m][i] = silu(g) * u,  silu(g) = g / (1 + exp(-g)),
    all in float64.  Returns float64 [len(rows)][I] (before rounding)."""
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
    rank rk, zero included ("ep_signal_completion": the value published for
    this expert; reading: the row count)."""
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
    description: without rank-level completion the destination checks each
    per-expert signal individually).  Reading: a word is ready when it carries
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

def combine_tokens(topk_ids, topk_w, recv_bufs, *, n_experts_per_device, my_rank,
                   top_k, msg_bytes, n, tokens=None, slot_row=None):
    """Top-k routing-weighted combine of the slots this GPU's experts wrote
    ("P3PeerSendConfig": the combine kernel reads slot (t, k) of rank rk;
    "ep_signal_completion": the consumer reads once the rank flag is set).

    out[rk][t][:] = bf16( sum over k = 0..top_k-1 whose expert is local of
    topk_w[rk][t][k] * slot(rk, t, k)[:] ), summed in float64 and rounded once;
    a token with no local pick gets +0.  ``tokens`` is an optional list of
    (rk, t) pairs; ``slot_row(rk, t, k)`` optionally supplies the bf16 codes of
    a slot instead of reading ``recv_bufs``.  Returns uint16 bf16 codes
    [len(tokens)][n] (or [R][T][n])."""
    ids = np.asarray(topk_ids)
    R, T, _ = ids.shape
    lo = my_rank * n_experts_per_device
    if slot_row is None:
        def slot_row(rk, t, k):
            off = recv_slot_offset(t, k, 0, top_k, msg_bytes)
            return recv_bufs[rk][off:off + 2 * n].view("<u2")
    pairs = ([(rk, t) for rk in range(R) for t in range(T)] if tokens is None
             else [(int(a), int(b)) for a, b in tokens])
    out = np.zeros((len(pairs), n), dtype=np.float64)
    for i, (rk, t) in enumerate(pairs):
        acc = np.zeros(n, dtype=np.float64)
        for k in range(top_k):
            g = int(ids[rk, t, k])
            if not (lo <= g < lo + n_experts_per_device):
                continue
            acc = acc + float(topk_w[rk, t, k]) * bf16_to_f64(slot_row(rk, t, k))
        out[i] = acc
    bits = f64_to_bf16(out)
    return bits.reshape(R, T, n) if tokens is None else bits


def sampled_step(*, topk_ids, topk_w, x, w, n_ranks, n_experts_per_device, top_k,
                 msg_bytes, max_tokens_per_rank, my_rank=0, dtype="bf16", x_scale=None,
                 w_scale=None, rows=(), tokens=()):
    """The step's results on a sample, for shapes too large to run whole: the
    grouping and counts in full, the sent bf16 row of each row in ``rows``, and
    the combined output of each (rk, t) in ``tokens`` (whose local picks' rows
    are computed on the way).  Same definitions as run_step."""
    offsets, src_info = group_local_picks(topk_ids, n_experts_per_device, my_rank)
    row_of = {}
    for m in range(int(offsets[-1])):
        _, rk = row_owner(offsets, n_ranks, m)
        row_of[(rk, int(src_info[m][0]), int(src_info[m][1]))] = m
    lo = my_rank * n_experts_per_device
    need = set(int(m) for m in rows)
    for rk, t in tokens:
        for k in range(top_k):
            if lo <= int(topk_ids[rk, t, k]) < lo + n_experts_per_device:
                need.add(row_of[(int(rk), int(t), k)])
    need = np.array(sorted(need), dtype=np.int64)
    if dtype == "bf16":
        y = expert_rows_bf16_f64(x, w, offsets, n_ranks, need)
    else:
        y = expert_rows_fp8_f64(x, x_scale, w, w_scale, offsets, n_ranks, need)
    y_bits = {int(m): b for m, b in zip(need, f64_to_bf16(y))}
    out = combine_tokens(topk_ids, topk_w, None, n_experts_per_device=n_experts_per_device,
                         my_rank=my_rank, top_k=top_k, msg_bytes=msg_bytes, n=w.shape[1],
                         tokens=list(tokens),
                         slot_row=lambda rk, t, k: y_bits[row_of[(rk, t, k)]])
    return {"offsets": offsets, "src_info": src_info,
            "counts": recv_counts(offsets, n_ranks, n_experts_per_device),
            "row_bits": {int(m): y_bits[int(m)] for m in rows}, "out_bits": out}


# ---------------------------------------------------------------- whole step

def run_step(*, topk_ids, topk_w, x, w, n_ranks, n_experts_per_device, top_k,
             msg_bytes, max_tokens_per_rank, my_rank=0, dtype="bf16",
             x_scale=None, w_scale=None, epoch=1, sentinel=0xFF, per_expert=False):
    """One EP-combine step on this GPU's share, from routing to combined output.

    The grouped row layout is re-derived here from ``topk_ids``; ``x`` must be
    the expert input rows in that order ([M][K]).  Receive buffers start filled
    with ``sentinel`` bytes.  Returns a dict with the grouping, the rounded
    expert outputs, the receive buffers, the control state, the combined output
    (uint16 bf16 codes [R][T][N]) and the error bits."""
    offsets, src_info = group_local_picks(topk_ids, n_experts_per_device, my_rank)
    M = int(offsets[-1])
    if x.shape[0] != M:
        raise ValueError(f"x has {x.shape[0]} rows, routing gives {M}")
    if dtype == "bf16":
        y = expert_rows_bf16_f64(x, w, offsets, n_ranks)
    elif dtype == "fp8":
        y = expert_rows_fp8_f64(x, x_scale, w, w_scale, offsets, n_ranks)
    else:
        raise ValueError(dtype)
    y_bits = f64_to_bf16(y)
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
    return {"offsets": offsets, "src_info": src_info, "y": y, "y_bits": y_bits,
            "recv_bufs": recv, "control": ctrl, "out_bits": out, "err": err}

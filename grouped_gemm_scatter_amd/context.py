"""Device-buffer plumbing around the C ABI: allocates the receive buffers,
count/flag words, election and tile counters and the error word with torch,
creates the library handle and counts step epochs.  Every computation is a
call into the HIP library."""
from __future__ import annotations

import torch

from . import binding as B


class EpCombine:
    def __init__(self, *, n_ranks: int, top_k: int, max_tokens_per_rank: int,
                 n_experts_per_device: int, hidden_k: int, hidden_n: int,
                 my_rank: int = 0, msg_bytes: int | None = None, dtype: str = "bf16",
                 system_scope: bool = False, per_expert_release: bool = False,
                 epilogue_only: bool = False, flag_spin_limit: int = 0,
                 w_slice_major: bool = False, device_epoch: bool = False,
                 send_waves: int = 0, send_tile: bool = False,
                 sentinel: int | None = None, trace_records: int = 0, device=None):
        self.device = torch.device(device or "cuda")
        self.n_ranks, self.top_k = n_ranks, top_k
        self.max_tokens_per_rank = max_tokens_per_rank
        self.n_experts_per_device = n_experts_per_device
        self.hidden_k, self.hidden_n = hidden_k, hidden_n
        self.msg_bytes = msg_bytes or 2 * hidden_n
        self.my_rank = my_rank
        self.dtype = dtype
        self.per_expert_release = per_expert_release
        # the down-projection reads W as [E_l][K/64][N][64] (see pack_weights)
        self.w_slice_major = w_slice_major
        # the step's epoch lives in device memory (EP_FLAG_DEVICE_EPOCH): a step
        # captured in a HIP graph advances it on the device at every replay
        self.device_epoch = device_epoch
        # dedicated send waves (4) above the GEMM's MFMA waves, or their 128 x 128
        # tile with the sink inside the MFMA waves (send_tile)
        self.send_waves, self.send_tile = send_waves, send_tile
        self.epoch_word = (torch.zeros(1, dtype=torch.int64, device=self.device)
                           if device_epoch else None)
        cap = max_tokens_per_rank * top_k * self.msg_bytes
        if sentinel is None:
            self.recv = [torch.empty(cap, dtype=torch.uint8, device=self.device)
                         for _ in range(n_ranks)]
        else:
            self.recv = [torch.full((cap,), sentinel, dtype=torch.uint8, device=self.device)
                         for _ in range(n_ranks)]
        self.words = torch.zeros(n_experts_per_device * n_ranks + n_ranks, dtype=torch.int64,
                                 device=self.device)
        self.rank_counter = torch.zeros(n_ranks, dtype=torch.int32, device=self.device)
        self.tile_counter = torch.zeros(n_experts_per_device, dtype=torch.int32, device=self.device)
        self.error_word = torch.zeros(1, dtype=torch.int32, device=self.device)
        # tile trace records (EP_FLAG_TRACE), four int64 words each
        self.trace = (torch.zeros((trace_records, 4), dtype=torch.int64, device=self.device)
                      if trace_records > 0 else None)
        self.params = B.make_params(
            n_ranks=n_ranks, my_rank=my_rank, top_k=top_k, msg_bytes=self.msg_bytes,
            max_tokens_per_rank=max_tokens_per_rank, n_experts_per_device=n_experts_per_device,
            hidden_k=hidden_k, hidden_n=hidden_n,
            dtype=B.EP_DTYPE_FP8_E4M3_B128 if dtype == "fp8" else B.EP_DTYPE_BF16,
            flags=(B.EP_FLAG_SYSTEM_SCOPE if system_scope else 0)
            | (B.EP_FLAG_PER_EXPERT_RELEASE if per_expert_release else 0)
            | (B.EP_FLAG_EPILOGUE_ONLY if epilogue_only else 0)
            | (B.EP_FLAG_TRACE if self.trace is not None else 0)
            | (B.EP_FLAG_W_SLICE_MAJOR if w_slice_major else 0)
            | (B.EP_FLAG_DEVICE_EPOCH if device_epoch else 0)
            | (B.EP_FLAG_SEND_TILE if send_tile else 0),
            flag_spin_limit=flag_spin_limit, send_waves=send_waves)
        self.handle = B.ep_combine_init(self.params, self.recv, self.words, self.rank_counter,
                                        self.tile_counter, self.error_word, self.trace,
                                        self.epoch_word)
        self.epoch = 0

    # views of the control words
    @property
    def counts(self) -> torch.Tensor:
        return self.words[: self.n_experts_per_device * self.n_ranks]

    @property
    def flags(self) -> torch.Tensor:
        return self.words[self.n_experts_per_device * self.n_ranks:]

    def next_epoch(self, stream=None) -> int:
        """Starts a step: the next epoch.  With a device epoch this launches its
        advance on the stream (and ``self.epoch`` follows it on the host for the
        eager caller; inside a captured graph only the device word moves)."""
        self.epoch += 1
        if self.device_epoch:
            if self.epoch & 0xFFFFFFFF == 0:
                self.epoch += 1
            B.ep_advance_epoch(self.handle, stream)
        return self.epoch

    def _epoch(self, epoch):
        """The epoch argument of a call: 0 with a device epoch (the kernels read it)."""
        if self.device_epoch:
            return 0
        return self.epoch if epoch is None else epoch

    def _need(self, t, name: str, elems: int, elem_bytes: int):
        """Raises unless device tensor `t` holds at least `elems` elements of
        `elem_bytes` bytes each: the kernels read and write by pointer only,
        so a short or mistyped tensor would otherwise be read past its end."""
        if t is None or isinstance(t, int):
            return
        if t.element_size() != elem_bytes:
            raise ValueError(f"{name}: {elem_bytes}-byte elements expected for this handle "
                             f"({self.dtype}), got {t.dtype}")
        if t.numel() < elems:
            raise ValueError(f"{name}: {t.numel()} elements, at least {elems} needed")

    def gemm_scatter(self, x, w, offsets, src_info, m_total, *, x_scale=None, w_scale=None,
                     p3_control: int = 0, c_local=None, epoch: int | None = None, stream=None,
                     noalloc: bool = False):
        """Grouped GEMM + row scatter + completion; ``noalloc`` calls the
        allocation-free entry point (library-held counters)."""
        K, N, El, R = self.hidden_k, self.hidden_n, self.n_experts_per_device, self.n_ranks
        eb = 1 if self.dtype == "fp8" else 2
        self._need(x, "x", m_total * K, eb)
        self._need(w, "w", El * N * K, eb)
        self._need(offsets, "offsets", El * R + 1, 4)
        self._need(src_info, "src_info", 2 * m_total, 4)
        if self.dtype == "fp8":
            self._need(x_scale, "x_scale", m_total * (K // 128), 4)
            self._need(w_scale, "w_scale", El * (N // 128) * (K // 128), 4)
        if p3_control < 0:
            self._need(c_local, "c_local", m_total * N, 2)
        return B.ep_grouped_gemm_scatter(
            self.handle, x, w, x_scale, w_scale, offsets, src_info, m_total, p3_control,
            c_local, self._epoch(epoch), stream, noalloc=noalloc)

    def gemm_tile(self, m_total: int) -> tuple:
        """(tile kind, rows, columns) of the grouped GEMM for m_total rows."""
        return B.ep_gemm_tile(self.handle, m_total)

    def signal(self, expert, dst_rank, signal, epoch: int | None = None, stream=None):
        return B.ep_signal_completion(self.handle, expert, dst_rank, signal, expert.numel(),
                                      self._epoch(epoch), stream)

    def group(self, topk_ids, *, offsets=None, src_info=None, stream=None):
        """Local grouping of the routing topk_ids [R][T][top_k] (int32 global
        expert ids): returns (offsets [E_l*R + 1], src_info [R*T*top_k][2]),
        both int32 on the device; rows [0, offsets[-1]) of src_info are the
        grouped (t, k) of the local picks."""
        R, T, k = topk_ids.shape
        if R != self.n_ranks or k != self.top_k:
            raise ValueError(f"topk_ids must be [{self.n_ranks}][T][{self.top_k}]")
        if offsets is None:
            offsets = torch.empty(self.n_experts_per_device * R + 1, dtype=torch.int32,
                                  device=self.device)
        if src_info is None:
            src_info = torch.empty((R * T * k, 2), dtype=torch.int32, device=self.device)
        self._need(topk_ids, "topk_ids", R * T * k, 4)
        self._need(offsets, "offsets", self.n_experts_per_device * R + 1, 4)
        self._need(src_info, "src_info", 2 * R * T * k, 4)
        B.ep_group_local_picks(self.handle, topk_ids, T, offsets, src_info, stream)
        return offsets, src_info

    def dispatch(self, tokens_x, offsets, src_info, m_total, x_out, *, stream=None):
        """Dispatch side: x_out[m] = tokens_x[rk][t] for every grouped row m
        (tokens_x [R][T][row] and x_out [M][row], any element type)."""
        R, T = tokens_x.shape[0], tokens_x.shape[1]
        row_bytes = tokens_x[0, 0].numel() * tokens_x.element_size()
        if R != self.n_ranks:
            raise ValueError(f"tokens_x must have {self.n_ranks} source ranks")
        if m_total and x_out.numel() * x_out.element_size() < m_total * row_bytes:
            raise ValueError("x_out is too small")
        self._need(offsets, "offsets", self.n_experts_per_device * self.n_ranks + 1, 4)
        self._need(src_info, "src_info", 2 * m_total, 4)
        return B.ep_dispatch_rows(self.handle, tokens_x, T, row_bytes, offsets, src_info, m_total,
                                  x_out, stream)

    def pack_weights(self, w, *, out=None, stream=None):
        """W [E_l][N][K] bf16 re-laid as [E_l][K/64][N][64] (a new tensor
        unless `out` is given): the layout a handle made with
        w_slice_major=True multiplies by."""
        n = self.n_experts_per_device * self.hidden_n * self.hidden_k
        self._need(w, "w", n, 2)
        if out is None:
            out = torch.empty((self.n_experts_per_device, self.hidden_k // 64, self.hidden_n, 64),
                              dtype=torch.bfloat16, device=self.device)
        self._need(out, "out", n, 2)
        B.ep_pack_weights(self.handle, w, out, stream)
        return out

    def up_swiglu(self, x1, w1, offsets, m_total, h_out, *, stream=None):
        """The expert FFN's first GEMM with SwiGLU: h_out [M][hidden_k] from
        x1 [M][hidden_n] and w1 [E_l][2*hidden_k][hidden_n] (gate rows, then up)."""
        hid, inter = self.hidden_n, self.hidden_k
        self._need(x1, "x1", m_total * hid, 2)
        self._need(w1, "w1", self.n_experts_per_device * 2 * inter * hid, 2)
        self._need(offsets, "offsets", self.n_experts_per_device * self.n_ranks + 1, 4)
        self._need(h_out, "h_out", m_total * inter, 2)
        return B.ep_grouped_gemm_swiglu(self.handle, x1, w1, offsets, m_total, h_out, stream)

    def up_swiglu_fp8(self, x1, x1_scale, w1, w1_scale, offsets, m_total, h_out, h_scale, *,
                      stream=None):
        """The fp8 expert FFN's first GEMM with SwiGLU: h_out [M][hidden_k] e4m3fn
        codes and h_scale [M][hidden_k/128] from x1 [M][hidden_n] (+ x1_scale
        [M][hidden_n/128]) and w1 [E_l][2*hidden_k][hidden_n] (+ w1_scale
        [E_l][2*hidden_k/128][hidden_n/128]), gate rows then up rows."""
        hid, inter, El = self.hidden_n, self.hidden_k, self.n_experts_per_device
        self._need(x1, "x1", m_total * hid, 1)
        self._need(x1_scale, "x1_scale", m_total * (hid // 128), 4)
        self._need(w1, "w1", El * 2 * inter * hid, 1)
        self._need(w1_scale, "w1_scale", El * (2 * inter // 128) * (hid // 128), 4)
        self._need(offsets, "offsets", El * self.n_ranks + 1, 4)
        self._need(h_out, "h_out", m_total * inter, 1)
        self._need(h_scale, "h_scale", m_total * (inter // 128), 4)
        return B.ep_grouped_gemm_swiglu_fp8(self.handle, x1, x1_scale, w1, w1_scale, offsets,
                                            m_total, h_out, h_scale, stream)

    def combine(self, topk_ids, topk_w, out, *, tokens_per_rank: int | None = None,
                epoch: int | None = None, stream=None):
        t = topk_ids.shape[1] if tokens_per_rank is None else tokens_per_rank
        self._need(topk_ids, "topk_ids", self.n_ranks * t * self.top_k, 4)
        self._need(topk_w, "topk_w", self.n_ranks * t * self.top_k, 4)
        self._need(out, "out", self.n_ranks * t * self.hidden_n, 2)
        return B.ep_combine_reduce(self.handle, topk_ids, topk_w, t, out,
                                   self._epoch(epoch), stream)

    def step(self, x, w, offsets, src_info, m_total, topk_ids, topk_w, out, *, x_scale=None,
             w_scale=None, stream=None, fused: bool = False):
        """One EP-combine step: grouped GEMM + scatter + signals, then combine
        (two launches, or one with ``fused``: ep_grouped_gemm_scatter_combine)."""
        self.next_epoch(stream)
        if fused:
            self.gemm_scatter_combine(x, w, offsets, src_info, m_total, topk_ids, topk_w, out,
                                      x_scale=x_scale, w_scale=w_scale, stream=stream)
            return
        self.gemm_scatter(x, w, offsets, src_info, m_total, x_scale=x_scale, w_scale=w_scale,
                          stream=stream)
        self.combine(topk_ids, topk_w, out, stream=stream)

    def gemm_scatter_combine(self, x, w, offsets, src_info, m_total, topk_ids, topk_w, out, *,
                             x_scale=None, w_scale=None, tokens_per_rank: int | None = None,
                             epoch: int | None = None, stream=None):
        """The whole step in one launch (consumer in the GEMM's grid)."""
        K, N, El, R = self.hidden_k, self.hidden_n, self.n_experts_per_device, self.n_ranks
        eb = 1 if self.dtype == "fp8" else 2
        t = topk_ids.shape[1] if tokens_per_rank is None else tokens_per_rank
        self._need(x, "x", m_total * K, eb)
        self._need(w, "w", El * N * K, eb)
        self._need(offsets, "offsets", El * R + 1, 4)
        self._need(src_info, "src_info", 2 * m_total, 4)
        if self.dtype == "fp8":
            self._need(x_scale, "x_scale", m_total * (K // 128), 4)
            self._need(w_scale, "w_scale", El * (N // 128) * (K // 128), 4)
        self._need(topk_ids, "topk_ids", R * t * self.top_k, 4)
        self._need(topk_w, "topk_w", R * t * self.top_k, 4)
        self._need(out, "out", R * t * N, 2)
        return B.ep_grouped_gemm_scatter_combine(
            self.handle, x, w, x_scale, w_scale, offsets, src_info, m_total, topk_ids, topk_w, t,
            out, self._epoch(epoch), stream)

    def reset_trace(self):
        """Zeroes the trace records (a slot with start clock 0 is unused)."""
        self.trace.zero_()

    def trace_table(self) -> dict:
        """The used trace records as host arrays: first row m0 and column n0,
        local expert, rows, cols, workgroup, start and end clocks (ticks of the
        device wall clock)."""
        import numpy as np
        r = self.trace.cpu().numpy().view(np.uint64)
        r = r[r[:, 2] != 0]
        w0, w1 = r[:, 0], r[:, 1]
        return {
            "m0": (w0 >> 32).astype(np.int64), "n0": (w0 & 0xffffffff).astype(np.int64),
            "expert": (w1 & 0xffff).astype(np.int64), "rows": ((w1 >> 16) & 0xffff).astype(np.int64),
            "cols": ((w1 >> 32) & 0xffff).astype(np.int64), "workgroup": (w1 >> 48).astype(np.int64),
            "t_start": r[:, 2].astype(np.int64), "t_end": r[:, 3].astype(np.int64),
        }

    def query_error(self, stream=None) -> int:
        return B.ep_combine_query_error(self.handle, stream)

    def close(self):
        if getattr(self, "handle", None):
            B.ep_combine_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

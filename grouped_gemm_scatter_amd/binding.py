"""ctypes binding of libep_combine.so (the C ABI in include/ep_combine.h).

Argument marshalling only: every step of the EP-combine path runs in the HIP
kernels of the library.  Functions keep the C names; device arguments are
torch tensors on the current HIP device (PyTorch supplies device memory and
streams), passed as raw pointers.  The library must have been built
(``python -m grouped_gemm_scatter_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_combine.so")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_UNSUPPORTED = -2
EP_ERR_HIP = -3
EP_ERR_SLOT_OOB = 0x1
EP_ERR_FLAG_TIMEOUT = 0x2
EP_ERR_BAD_GROUP = 0x4
EP_DTYPE_BF16 = 0
EP_DTYPE_FP8_E4M3_B128 = 1
EP_FLAG_SYSTEM_SCOPE = 0x1
EP_FLAG_PER_EXPERT_RELEASE = 0x2
EP_FLAG_EPILOGUE_ONLY = 0x4
EP_FLAG_TRACE = 0x8
EP_FLAG_W_SLICE_MAJOR = 0x10
EP_FLAG_DEVICE_EPOCH = 0x20
EP_FLAG_SEND_TILE = 0x40
EP_MAX_RANKS = 8

EXPORTED = ("ep_combine_init", "ep_combine_destroy", "ep_gemm_tile", "ep_group_local_picks",
            "ep_dispatch_rows", "ep_pack_weights", "ep_advance_epoch",
            "ep_grouped_gemm_scatter", "ep_grouped_gemm_scatter_noalloc", "ep_grouped_gemm_swiglu",
            "ep_grouped_gemm_swiglu_fp8",
            "ep_grouped_gemm_scatter_combine", "ep_signal_completion",
            "ep_combine_reduce", "ep_combine_query_error", "ep_combine_strerror",
            "ep_combine_version")


class EpCombineParams(ctypes.Structure):
    _fields_ = [
        ("n_ranks", ctypes.c_int32),
        ("p2p_world_size", ctypes.c_int32),
        ("my_rank", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("msg_bytes", ctypes.c_int32),
        ("max_tokens_per_rank", ctypes.c_int32),
        ("n_experts_per_device", ctypes.c_int32),
        ("hidden_k", ctypes.c_int32),
        ("hidden_n", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("send_waves", ctypes.c_int32),
        ("flag_spin_limit", ctypes.c_int64),
    ]


class EpCombineBuffers(ctypes.Structure):
    _fields_ = [
        ("recv_buf", ctypes.c_void_p * EP_MAX_RANKS),
        ("recv_count", ctypes.c_void_p),
        ("rank_counter", ctypes.c_void_p),
        ("tile_counter", ctypes.c_void_p),
        ("error_word", ctypes.c_void_p),
        ("trace", ctypes.c_void_p),
        ("trace_records", ctypes.c_int64),
        ("epoch_word", ctypes.c_void_p),
    ]


class EpError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def load_library(path: str | None = None):
    """Loads the HIP library once (torch is imported first so that the library
    binds to the HIP runtime torch already loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing; build it with "
            "`python -m grouped_gemm_scatter_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    lib.ep_combine_init.argtypes = [ctypes.POINTER(EpCombineParams),
                                    ctypes.POINTER(EpCombineBuffers), ctypes.POINTER(vp)]
    lib.ep_combine_init.restype = ctypes.c_int
    lib.ep_combine_destroy.argtypes = [vp]
    lib.ep_combine_destroy.restype = None
    lib.ep_grouped_gemm_scatter.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, u64, vp]
    lib.ep_grouped_gemm_scatter.restype = ctypes.c_int
    lib.ep_grouped_gemm_scatter_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                                    u64, vp]
    lib.ep_grouped_gemm_scatter_noalloc.restype = ctypes.c_int
    lib.ep_grouped_gemm_scatter_combine.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32,
                                                    vp, u64, vp]
    lib.ep_grouped_gemm_scatter_combine.restype = ctypes.c_int
    lib.ep_grouped_gemm_swiglu.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    lib.ep_grouped_gemm_swiglu_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.ep_grouped_gemm_swiglu_fp8.restype = ctypes.c_int
    lib.ep_grouped_gemm_swiglu.restype = ctypes.c_int
    lib.ep_gemm_tile.argtypes = [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.ep_gemm_tile.restype = ctypes.c_int
    lib.ep_group_local_picks.argtypes = [vp, vp, i32, vp, vp, vp]
    lib.ep_dispatch_rows.argtypes = [vp, vp, i32, i32, vp, vp, i32, vp, vp]
    lib.ep_dispatch_rows.restype = ctypes.c_int
    lib.ep_pack_weights.argtypes = [vp, vp, vp, vp]
    lib.ep_advance_epoch.argtypes = [vp, vp]
    lib.ep_advance_epoch.restype = ctypes.c_int
    lib.ep_pack_weights.restype = ctypes.c_int
    lib.ep_group_local_picks.restype = ctypes.c_int
    lib.ep_signal_completion.argtypes = [vp, vp, vp, vp, i32, u64, vp]
    lib.ep_signal_completion.restype = ctypes.c_int
    lib.ep_combine_reduce.argtypes = [vp, vp, vp, i32, vp, u64, vp]
    lib.ep_combine_reduce.restype = ctypes.c_int
    lib.ep_combine_query_error.argtypes = [vp, vp]
    lib.ep_combine_query_error.restype = ctypes.c_int
    lib.ep_combine_strerror.argtypes = [ctypes.c_int]
    lib.ep_combine_strerror.restype = ctypes.c_char_p
    lib.ep_combine_version.argtypes = []
    lib.ep_combine_version.restype = ctypes.c_int
    del i64
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().ep_combine_strerror(int(code)).decode()


def _ptr(t, dtype=None, name="tensor", allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise EpError(rc, what)
    return rc


def make_params(*, n_ranks, my_rank, top_k, msg_bytes, max_tokens_per_rank,
                n_experts_per_device, hidden_k, hidden_n, dtype=EP_DTYPE_BF16, flags=0,
                flag_spin_limit=0, p2p_world_size=None, send_waves=0) -> EpCombineParams:
    return EpCombineParams(n_ranks, n_ranks if p2p_world_size is None else p2p_world_size,
                           my_rank, top_k, msg_bytes, max_tokens_per_rank,
                           n_experts_per_device, hidden_k, hidden_n, dtype, flags, send_waves,
                           flag_spin_limit)


def ep_combine_init(params: EpCombineParams, recv_bufs, recv_count, rank_counter,
                    tile_counter, error_word, trace=None, epoch_word=None) -> int:
    """Returns an opaque handle (int).  Buffers are device tensors that must
    outlive the handle; `trace` is an int64 [records][4] tensor, used with
    EP_FLAG_TRACE only; `epoch_word` one int64, with EP_FLAG_DEVICE_EPOCH only."""
    lib = load_library()
    b = EpCombineBuffers()
    if len(recv_bufs) > EP_MAX_RANKS:
        raise ValueError("at most 8 receive buffers")
    for i, rb in enumerate(recv_bufs):
        b.recv_buf[i] = _ptr(rb, torch.uint8, f"recv_buf[{i}]")
    b.recv_count = _ptr(recv_count, (torch.int64, torch.uint64), "recv_count")
    b.rank_counter = _ptr(rank_counter, torch.int32, "rank_counter")
    b.tile_counter = _ptr(tile_counter, torch.int32, "tile_counter")
    b.error_word = _ptr(error_word, torch.int32, "error_word")
    if trace is not None:
        if trace.dim() != 2 or trace.shape[1] != 4:
            raise ValueError("trace must be [records][4]")
        b.trace = _ptr(trace, (torch.int64, torch.uint64), "trace")
        b.trace_records = trace.shape[0]
    if epoch_word is not None:
        b.epoch_word = _ptr(epoch_word, (torch.int64, torch.uint64), "epoch_word")
    h = ctypes.c_void_p()
    _check(lib.ep_combine_init(ctypes.byref(params), ctypes.byref(b), ctypes.byref(h)),
           "ep_combine_init")
    return h.value


def ep_combine_destroy(h: int) -> None:
    if h:
        load_library().ep_combine_destroy(h)


def ep_grouped_gemm_scatter(h, x, w, x_scale, w_scale, offsets, src_info, m_total,
                            p3_control=0, c_local=None, epoch=1, stream=None,
                            noalloc=False) -> int:
    """The GEMM + scatter call; ``noalloc`` selects the allocation-free entry
    point ep_grouped_gemm_scatter_noalloc (library-held counters)."""
    lib = load_library()
    name = "ep_grouped_gemm_scatter_noalloc" if noalloc else "ep_grouped_gemm_scatter"
    rc = getattr(lib, name)(
        h, _ptr(x, None, "x", allow_none=True), _ptr(w, None, "w"),
        _ptr(x_scale, torch.float32, "x_scale", allow_none=True),
        _ptr(w_scale, torch.float32, "w_scale", allow_none=True),
        _ptr(offsets, torch.int32, "offsets"),
        _ptr(src_info, torch.int32, "src_info", allow_none=True),
        int(m_total), int(p3_control), _ptr(c_local, torch.bfloat16, "c_local", allow_none=True),
        int(epoch), _stream(stream))
    return _check(rc, name)


def ep_grouped_gemm_scatter_combine(h, x, w, x_scale, w_scale, offsets, src_info, m_total,
                                    topk_ids, topk_w, tokens_per_rank, out, epoch=1,
                                    stream=None) -> int:
    lib = load_library()
    rc = lib.ep_grouped_gemm_scatter_combine(
        h, _ptr(x, None, "x", allow_none=True), _ptr(w, None, "w"),
        _ptr(x_scale, torch.float32, "x_scale", allow_none=True),
        _ptr(w_scale, torch.float32, "w_scale", allow_none=True),
        _ptr(offsets, torch.int32, "offsets"),
        _ptr(src_info, torch.int32, "src_info", allow_none=True), int(m_total),
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        int(tokens_per_rank), _ptr(out, torch.bfloat16, "out"), int(epoch), _stream(stream))
    return _check(rc, "ep_grouped_gemm_scatter_combine")


def ep_gemm_tile(h, m_total) -> tuple:
    """(tile kind, tile rows, tile columns) ep_grouped_gemm_scatter uses for
    m_total rows on handle h."""
    lib = load_library()
    r, c = ctypes.c_int32(), ctypes.c_int32()
    kind = _check(lib.ep_gemm_tile(h, int(m_total), ctypes.byref(r), ctypes.byref(c)),
                  "ep_gemm_tile")
    return kind, r.value, c.value


def ep_dispatch_rows(h, tokens_x, tokens_per_rank, row_bytes, offsets, src_info, m_total,
                     x_out, stream=None) -> int:
    lib = load_library()
    rc = lib.ep_dispatch_rows(h, _ptr(tokens_x, None, "tokens_x", allow_none=True),
                              int(tokens_per_rank), int(row_bytes),
                              _ptr(offsets, torch.int32, "offsets"),
                              _ptr(src_info, torch.int32, "src_info", allow_none=True),
                              int(m_total), _ptr(x_out, None, "x_out", allow_none=True),
                              _stream(stream))
    return _check(rc, "ep_dispatch_rows")


def ep_advance_epoch(h, stream=None) -> int:
    lib = load_library()
    return _check(lib.ep_advance_epoch(h, _stream(stream)), "ep_advance_epoch")


def ep_pack_weights(h, w, w_out, stream=None) -> int:
    lib = load_library()
    rc = lib.ep_pack_weights(h, _ptr(w, torch.bfloat16, "w"), _ptr(w_out, torch.bfloat16, "w_out"),
                             _stream(stream))
    return _check(rc, "ep_pack_weights")


def ep_group_local_picks(h, topk_ids, tokens_per_rank, offsets, src_info, stream=None) -> int:
    lib = load_library()
    rc = lib.ep_group_local_picks(h, _ptr(topk_ids, torch.int32, "topk_ids", allow_none=True),
                                  int(tokens_per_rank), _ptr(offsets, torch.int32, "offsets"),
                                  _ptr(src_info, torch.int32, "src_info", allow_none=True),
                                  _stream(stream))
    return _check(rc, "ep_group_local_picks")


def ep_grouped_gemm_swiglu(h, x1, w1, offsets, m_total, h_out, stream=None) -> int:
    lib = load_library()
    rc = lib.ep_grouped_gemm_swiglu(
        h, _ptr(x1, torch.bfloat16, "x1", allow_none=True), _ptr(w1, torch.bfloat16, "w1"),
        _ptr(offsets, torch.int32, "offsets"), int(m_total),
        _ptr(h_out, torch.bfloat16, "h_out", allow_none=True), _stream(stream))
    return _check(rc, "ep_grouped_gemm_swiglu")


def ep_grouped_gemm_swiglu_fp8(h, x1, x1_scale, w1, w1_scale, offsets, m_total, h_out, h_scale,
                               stream=None) -> int:
    lib = load_library()
    rc = lib.ep_grouped_gemm_swiglu_fp8(
        h, _ptr(x1, torch.uint8, "x1", allow_none=True),
        _ptr(x1_scale, torch.float32, "x1_scale", allow_none=True), _ptr(w1, torch.uint8, "w1"),
        _ptr(w1_scale, torch.float32, "w1_scale"), _ptr(offsets, torch.int32, "offsets"),
        int(m_total), _ptr(h_out, torch.uint8, "h_out", allow_none=True),
        _ptr(h_scale, torch.float32, "h_scale", allow_none=True), _stream(stream))
    return _check(rc, "ep_grouped_gemm_swiglu_fp8")


def ep_signal_completion(h, expert, dst_rank, signal, n, epoch, stream=None) -> int:
    lib = load_library()
    rc = lib.ep_signal_completion(h, _ptr(expert, torch.int32, "expert", allow_none=True),
                                  _ptr(dst_rank, torch.int32, "dst_rank", allow_none=True),
                                  _ptr(signal, (torch.int64, torch.uint64), "signal",
                                       allow_none=True),
                                  int(n), int(epoch), _stream(stream))
    return _check(rc, "ep_signal_completion")


def ep_combine_reduce(h, topk_ids, topk_w, tokens_per_rank, out, epoch, stream=None) -> int:
    lib = load_library()
    rc = lib.ep_combine_reduce(h, _ptr(topk_ids, torch.int32, "topk_ids"),
                               _ptr(topk_w, torch.float32, "topk_w"), int(tokens_per_rank),
                               _ptr(out, torch.bfloat16, "out"), int(epoch), _stream(stream))
    return _check(rc, "ep_combine_reduce")


def ep_combine_query_error(h, stream=None) -> int:
    return _check(load_library().ep_combine_query_error(h, _stream(stream)),
                  "ep_combine_query_error")


def ep_combine_strerror(code: int) -> str:
    return strerror(code)


def ep_combine_version() -> int:
    return load_library().ep_combine_version()

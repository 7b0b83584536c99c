"""MI355X (gfx950) MoE expert-parallel combine: grouped GEMM whose epilogue
sends each output row to its owner's receive buffer, rank-level completion
signalling, and the top-k weighted combine.  The work runs in the HIP library
libep_combine.so (C ABI: include/ep_combine.h); this package is its ctypes
binding plus device-buffer plumbing."""
from .binding import (EP_DTYPE_BF16, EP_DTYPE_FP8_E4M3_B128, EP_ERR_BAD_GROUP,
                      EP_ERR_FLAG_TIMEOUT, EP_ERR_HIP, EP_ERR_INVALID_ARG, EP_ERR_SLOT_OOB,
                      EP_ERR_UNSUPPORTED, EP_FLAG_EPILOGUE_ONLY, EP_FLAG_PER_EXPERT_RELEASE,
                      EP_FLAG_SYSTEM_SCOPE, EP_FLAG_TRACE, EP_FLAG_W_SLICE_MAJOR, EP_FLAG_DEVICE_EPOCH, EP_FLAG_SEND_TILE, EP_OK, EpError,
                      ep_combine_destroy, ep_combine_init, ep_combine_query_error,
                      ep_combine_reduce, ep_combine_strerror, ep_combine_version,
                      ep_group_local_picks, ep_pack_weights,
                      ep_grouped_gemm_scatter, ep_grouped_gemm_swiglu, ep_signal_completion,
                      load_library, make_params)
from .context import EpCombine

__all__ = [
    "EP_DTYPE_BF16", "EP_DTYPE_FP8_E4M3_B128", "EP_ERR_BAD_GROUP", "EP_ERR_FLAG_TIMEOUT",
    "EP_ERR_HIP", "EP_ERR_INVALID_ARG", "EP_ERR_SLOT_OOB", "EP_ERR_UNSUPPORTED",
    "EP_FLAG_EPILOGUE_ONLY", "EP_FLAG_PER_EXPERT_RELEASE", "EP_FLAG_SYSTEM_SCOPE",
    "EP_FLAG_TRACE", "EP_FLAG_W_SLICE_MAJOR", "EP_FLAG_DEVICE_EPOCH", "EP_FLAG_SEND_TILE", "EP_OK", "EpError", "ep_combine_destroy", "ep_combine_init",
    "ep_combine_query_error", "ep_combine_reduce", "ep_combine_strerror",
    "ep_combine_version", "ep_group_local_picks", "ep_grouped_gemm_scatter", "ep_pack_weights",
    "ep_grouped_gemm_swiglu",
    "ep_signal_completion",
    "load_library", "make_params", "EpCombine",
]

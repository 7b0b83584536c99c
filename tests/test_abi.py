"""The C-ABI library loads and exports every symbol include/ep_combine.h
declares; host-side argument validation (no GPU work) and error strings."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_combine.h")


@pytest.fixture(scope="module")
def lib():
    from grouped_gemm_scatter_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from grouped_gemm_scatter_amd.build import build
        build(jobs=4)
    return binding.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"EP_API\s+[\w\s\*]+?\b(ep_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("ep_combine_init", "ep_grouped_gemm_scatter", "ep_signal_completion",
              "ep_combine_reduce"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from grouped_gemm_scatter_amd import binding
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(binding.EXPORTED) == _declared()


def test_library_is_built_for_gfx950():
    from grouped_gemm_scatter_amd import binding
    data = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_missing_library_fails_loudly(tmp_path):
    from grouped_gemm_scatter_amd import binding
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            binding.load_library(str(tmp_path / "nope.so"))
    finally:
        binding._lib = saved


def _init(lib, trace=None, trace_records=0, **over):
    from grouped_gemm_scatter_amd import binding as B
    kw = dict(n_ranks=2, my_rank=0, top_k=2, msg_bytes=256, max_tokens_per_rank=8,
              n_experts_per_device=2, hidden_k=64, hidden_n=128)
    kw.update(over)
    p = B.make_params(**kw)
    b = B.EpCombineBuffers()
    for i in range(kw["n_ranks"] if kw["n_ranks"] <= 8 else 8):
        b.recv_buf[i] = 4096 * (i + 1)
    b.recv_count = b.rank_counter = b.tile_counter = b.error_word = 1 << 20
    b.trace, b.trace_records = trace, trace_records
    h = ctypes.c_void_p()
    return lib.ep_combine_init(ctypes.byref(p), ctypes.byref(b), ctypes.byref(h))


@pytest.mark.parametrize("over,code", [
    (dict(n_ranks=9), -1), (dict(n_ranks=0), -1), (dict(my_rank=2), -1),
    (dict(top_k=0), -1), (dict(top_k=65), -1), (dict(n_experts_per_device=0), -1),
    (dict(n_experts_per_device=257), -1), (dict(msg_bytes=255), -1), (dict(msg_bytes=200), -1),
    (dict(hidden_n=96, msg_bytes=192), -2), (dict(hidden_k=96), -2), (dict(dtype=7), -2),
    (dict(dtype=1, hidden_k=192), -2), (dict(p2p_world_size=1), -2), (dict(flags=0x80), -1), (dict(flags=0x20), -1),
    (dict(dtype=1, hidden_k=128, flags=0x10), -2),
    # send waves: 0 or 4, bf16 only, no measurement modes
    (dict(send_waves=2), -1), (dict(send_waves=-4), -1),
    (dict(send_waves=4, dtype=1, hidden_k=128), -2), (dict(send_waves=4, flags=0x4), -2),
    (dict(flags=0x40, dtype=1, hidden_k=128), -2), (dict(flags=0x40 | 0x8), -2),
    (dict(flag_spin_limit=-1), -1),
])
def test_init_rejects_bad_geometry_on_the_host(lib, over, code):
    assert _init(lib, **over) == code


@pytest.mark.parametrize("trace,records", [(None, 16), (1 << 20, 0), (1 << 20, -4),
                                           ((1 << 20) + 8, 16)])
def test_init_rejects_unusable_trace_buffers(lib, trace, records):
    """EP_FLAG_TRACE needs a 16-byte aligned buffer of at least one record."""
    from grouped_gemm_scatter_amd import binding as B
    assert _init(lib, trace=trace, trace_records=records, flags=B.EP_FLAG_TRACE) == -1


def test_init_rejects_misaligned_receive_buffer(lib):
    from grouped_gemm_scatter_amd import binding as B
    p = B.make_params(n_ranks=1, my_rank=0, top_k=2, msg_bytes=256, max_tokens_per_rank=8,
                      n_experts_per_device=2, hidden_k=64, hidden_n=128)
    b = B.EpCombineBuffers()
    b.recv_buf[0] = 4096 + 8
    b.recv_count = b.rank_counter = b.tile_counter = b.error_word = 1 << 20
    h = ctypes.c_void_p()
    assert lib.ep_combine_init(ctypes.byref(p), ctypes.byref(b), ctypes.byref(h)) == -1


def test_null_handle_calls_are_rejected(lib):
    assert lib.ep_grouped_gemm_scatter(None, None, None, None, None, None, None, 0, 0, None, 1,
                                       None) == -1
    assert lib.ep_signal_completion(None, None, None, None, 1, 1, None) == -1
    assert lib.ep_combine_reduce(None, None, None, 1, None, 1, None) == -1
    assert lib.ep_combine_query_error(None, None) == -1
    assert lib.ep_group_local_picks(None, None, 0, None, None, None) == -1
    assert lib.ep_dispatch_rows(None, None, 0, 16, None, None, 0, None, None) == -1
    assert lib.ep_pack_weights(None, None, None, None) == -1
    assert lib.ep_advance_epoch(None, None) == -1
    assert lib.ep_grouped_gemm_swiglu(None, None, None, None, 0, None, None) == -1
    assert lib.ep_grouped_gemm_scatter_combine(None, None, None, None, None, None, None, 0, None,
                                               None, 0, None, 1, None) == -1
    assert lib.ep_grouped_gemm_scatter_noalloc(None, None, None, None, None, None, None, 0, 0,
                                               None, 1, None) == -1
    lib.ep_combine_destroy(None)


def test_strerror_covers_every_code(lib):
    from grouped_gemm_scatter_amd import binding as B
    for c in (B.EP_OK, B.EP_ERR_INVALID_ARG, B.EP_ERR_UNSUPPORTED, B.EP_ERR_HIP, B.EP_ERR_SLOT_OOB,
              B.EP_ERR_FLAG_TIMEOUT, B.EP_ERR_BAD_GROUP, 3, -99):
        s = B.strerror(c)
        assert isinstance(s, str) and s
    assert lib.ep_combine_version() >= 100

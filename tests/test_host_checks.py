"""Host-side operand checks of the device-buffer plumbing: a tensor too short
for the handle's shapes, or with elements of the wrong width for its dtype, is
rejected before anything is launched."""
import types

import pytest
import torch

from grouped_gemm_scatter_amd.context import EpCombine


def _fake(dtype):
    return types.SimpleNamespace(dtype=dtype)


def test_short_tensor_is_rejected():
    t = torch.zeros(99, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="at least 100"):
        EpCombine._need(_fake("bf16"), t, "x", 100, 2)
    EpCombine._need(_fake("bf16"), t, "x", 99, 2)


def test_wrong_element_width_is_rejected():
    # fp8 bytes reinterpreted as bf16 (half as many elements, twice as wide)
    b = torch.zeros(256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="2-byte elements"):
        EpCombine._need(_fake("bf16"), b, "x", 128, 2)
    with pytest.raises(ValueError, match="1-byte elements"):
        EpCombine._need(_fake("fp8"), b.view(torch.bfloat16), "x", 256, 1)
    EpCombine._need(_fake("fp8"), b, "x", 256, 1)


def test_absent_and_raw_pointer_operands_are_passed_through():
    EpCombine._need(_fake("bf16"), None, "c_local", 10, 2)
    EpCombine._need(_fake("bf16"), 0x1000, "x", 10, 2)

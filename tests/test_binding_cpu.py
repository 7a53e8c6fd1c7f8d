"""The Python wrappers reject bad tensors before reaching the library (CPU
only: no device memory is touched)."""
import pytest
import torch

import variable_length_flashattention_amd as rra


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def test_forward_rejects_wrong_dtypes():
    with pytest.raises(TypeError):
        rra.varlen_attn_fwd(torch.zeros(4, 2, 64), bf16(4, 2, 64), bf16(4, 2, 64), i32(2), i32(2), 4, 0.1, True)
    with pytest.raises(TypeError):
        rra.varlen_attn_fwd(bf16(4, 2, 64), bf16(4, 2, 64), bf16(4, 2, 64), torch.zeros(2, dtype=torch.int64), i32(2),
                            4, 0.1, True)


def test_forward_rejects_host_tensors():
    with pytest.raises(ValueError):
        rra.varlen_attn_fwd(bf16(4, 2, 64), bf16(4, 2, 64), bf16(4, 2, 64), i32(2), i32(2), 4, 0.1, True)


def test_decode_rejects_bad_inputs():
    with pytest.raises(TypeError):
        rra.paged_decode_attn(torch.zeros(2, 4, 64), bf16(3, 16, 2, 64), bf16(3, 16, 2, 64), i32(2, 2), i32(2), 0.1)
    with pytest.raises(ValueError):  # host tensors
        rra.paged_decode_attn(bf16(2, 4, 64), bf16(3, 16, 2, 64), bf16(3, 16, 2, 64), i32(2, 2), i32(2), 0.1)


def test_paged_forward_and_backward_reject_host_tensors():
    with pytest.raises(ValueError):
        rra.varlen_attn_fwd_paged(bf16(4, 2, 64), bf16(3, 16, 2, 64), bf16(3, 16, 2, 64), i32(2), i32(1), i32(1, 3),
                                  4, 0.1, True)
    with pytest.raises(ValueError):
        rra.varlen_attn_bwd(bf16(4, 2, 64), bf16(4, 2, 64), bf16(4, 2, 64), bf16(4, 2, 64), torch.zeros(4, 2),
                            bf16(4, 2, 64), i32(2), i32(2), 4, 4, 0.1, True)

"""Host-side checks of the autograd wrapper: it rejects what the kernels cannot take
before anything reaches the library, and never computes on the CPU."""
import pytest
import torch

from exact_attention_backward_fa_amd import attention


def _qkv(dtype=torch.float16):
    q = torch.zeros(1, 2, 8, 64, dtype=dtype, requires_grad=True)
    k = torch.zeros(1, 1, 8, 64, dtype=dtype, requires_grad=True)
    v = torch.zeros(1, 1, 8, 64, dtype=dtype, requires_grad=True)
    return q, k, v


def test_cpu_tensors_are_rejected():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="HIP device"):
        attention(q, k, v, causal=True)


def test_unknown_dq_mode_is_rejected():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="dq_mode"):
        attention(q, k, v, dq_mode="fastest")


def test_float32_is_rejected():
    q, k, v = _qkv(torch.float32)
    with pytest.raises(ValueError, match="float16 or bfloat16"):
        attention(q, k, v)


def test_wrong_rank_is_rejected():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="4-D"):
        attention(q[0], k, v)

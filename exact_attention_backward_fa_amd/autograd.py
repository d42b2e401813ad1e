"""PyTorch autograd wrapper over the C ABI: exact softmax attention whose forward
is ``fa_fwd`` and whose backward is ``fa_bwd``.

The Liger-Kernel flash-attention page ("[Kernel] Flash attention 2", its summary)
puts its kernel in place of the SDPA attention of existing model layers; this is
that integration layer for these kernels and nothing more: it saves the forward's O and its
per-row log-sum-exp for the backward (which needs both, as every page's backward
does) and hands dO to the backward kernels.  Arguments are marshalled only
(made contiguous); all arithmetic runs in the HIP kernels, and tensors that are not
on a HIP device are rejected.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib


class _ExactAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale: float, causal: bool, dq_mode: str):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = _lib.fwd(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal, ctx.dq_mode = scale, causal, dq_mode
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _lib.bwd(q, k, v, o, lse, do.contiguous(), ctx.scale, ctx.causal,
                              dq_mode=ctx.dq_mode)
        need = ctx.needs_input_grad
        return (dq if need[0] else None, dk if need[1] else None, dv if need[2] else None,
                None, None, None)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              scale: Optional[float] = None, dq_mode: str = "auto") -> torch.Tensor:
    """softmax(scale * q kᵀ [+ causal mask]) v, differentiable in q, k and v.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nkv, d] with Hq a multiple of Hkv (query head h
    reads kv head h // (Hq / Hkv)); float16 or bfloat16 on one HIP device; d in
    {64, 128}.  ``scale`` defaults to 1/sqrt(d).  The causal mask is aligned to the
    bottom-right corner: query i sees key j when j <= i + (Nkv - Nq).  ``dq_mode``
    picks the backward's dQ path ("auto", "atomic" or "separate").
    """
    if q.dim() != 4:
        raise ValueError("q must be 4-D [B, Hq, Nq, d]")
    s = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    if dq_mode not in _lib.DQ_MODES:
        raise ValueError(f"dq_mode must be one of {list(_lib.DQ_MODES)}")
    return _ExactAttention.apply(q, k, v, s, bool(causal), dq_mode)

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


class _BiasDropoutAttention(torch.autograd.Function):
    """fa_fwd_bias_dropout / fa_bwd_bias_dropout; the bias arrives expanded to
    [B, Hq, Nq, Nkv] (a view), so autograd sums its full gradient back over the
    dimensions it was broadcast along."""

    @staticmethod
    def forward(ctx, q, k, v, bias, scale: float, causal: bool, dropout_p: float, seed: int):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = _lib.fwd_bias_dropout(q, k, v, scale, causal, bias=bias, dropout_p=dropout_p,
                                       seed=seed)
        ctx.save_for_backward(q, k, v, o, lse, bias)
        ctx.scale, ctx.causal, ctx.dropout_p, ctx.seed = scale, causal, dropout_p, seed
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, bias = ctx.saved_tensors
        need = ctx.needs_input_grad
        dq, dk, dv, dbias = _lib.bwd_bias_dropout(q, k, v, o, lse, do.contiguous(), ctx.scale,
                                                  ctx.causal, bias=bias, want_dbias=need[3],
                                                  dropout_p=ctx.dropout_p, seed=ctx.seed)
        return (dq if need[0] else None, dk if need[1] else None, dv if need[2] else None,
                dbias, None, None, None, None)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              scale: Optional[float] = None, dq_mode: str = "auto",
              bias: Optional[torch.Tensor] = None, dropout_p: float = 0.0,
              seed: int = 0) -> torch.Tensor:
    """dropout(softmax(scale * q kᵀ + bias [+ causal mask])) v, differentiable in q, k,
    v and the bias.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nkv, d] with Hq a multiple of Hkv (query head h
    reads kv head h // (Hq / Hkv)); float16 or bfloat16 on one HIP device; d in
    {32, 64, ..., 256} (multiples of 32).  ``scale`` defaults to 1/sqrt(d).  The causal mask is
    aligned to the bottom-right corner: query i sees key j when j <= i + (Nkv - Nq).
    ``dq_mode`` picks the backward's dQ path ("auto", "atomic" or "separate").
    ``bias`` (q's dtype, 4-D, each dimension its full size or 1, rows 16-byte
    aligned) is added to the scaled scores; ``dropout_p`` drops probabilities with
    the library's Philox mask from ``seed`` (the same seed reproduces the same mask).
    With a bias or dropout the separate dQ path runs; a bias that is one value per
    (batch, key) and needs no gradient runs at every head dim, any other bias and
    dropout at d = 64 or 128.
    """
    if q.dim() != 4:
        raise ValueError("q must be 4-D [B, Hq, Nq, d]")
    s = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    if dq_mode not in _lib.DQ_MODES:
        raise ValueError(f"dq_mode must be one of {list(_lib.DQ_MODES)}")
    if bias is None and dropout_p == 0.0:
        return _ExactAttention.apply(q, k, v, s, bool(causal), dq_mode)
    if dq_mode == "atomic":
        raise ValueError("a bias or dropout runs on the separate dQ path")
    if bias is not None:
        B, Hq, Nq, _ = q.shape
        bias = bias.expand(B, Hq, Nq, k.shape[2])
    return _BiasDropoutAttention.apply(q, k, v, bias, s, bool(causal), float(dropout_p), int(seed))

"""torch.autograd entry point over the C-ABI kernels.

"Triton FlashAttention" wraps its kernels in an autograd function that saves
Q, K, V, O and the per-row log-sum-exp for the backward and refuses double
backward rather than computing it wrongly ("FlashAttention-2 from PyTorch to
Triton" does the same in its autograd function).  ``attention`` is that call:
the forward runs ``fa_fwd``, the backward ``fa_bwd``; nothing else is
computed here, and beyond the outputs the only memory held is O(B*H*S) (the
log-sum-exp, and the rowsum workspace during the backward).
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import fa

__all__ = ["attention"]


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = fa.fa_fwd(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    @once_differentiable
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, do, lse, ctx.causal, ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal=False, scale: float | None = None):
    """Exact scaled-dot-product attention of ``[B, H, S, D]`` tensors (any
    strides; fp16, bf16 or fp32 on one GPU), differentiable once.

    ``scale`` defaults to ``1/sqrt(D)``; ``causal`` is False (none), True or
    1 (key j visible to query i iff j <= i, top-left aligned), or 2 /
    "bottom_right" (j <= i + Sk - Sq; rows with no visible key give 0).
    """
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _Attention.apply(q, k, v, causal, float(scale))

"""Autograd node over the C ABI: the differentiable attention op.

The pages' framework exposes fused attention as one op whose backward node
keeps the forward's inputs, its output and the O(S) logsumexp L next to them
(T14 flash-attention design doc, "What flash-attention is" and Key Design
Decision 2: L is what lets the backward recompute P instead of storing it).
This is that node for PyTorch: `forward` runs xfa_fwd and saves
(q, k, v, out, L); `backward` runs xfa_bwd_preprocess and xfa_bwd.  Nothing of
size S x S is kept.  Every step runs in libxfa.so; there is no fallback.
"""

from __future__ import annotations

import math

import torch

from . import _binding as _b


class FlashAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, lse = _b.forward(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.scale, ctx.causal = scale, causal
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = _b.backward(q, k, v, out, dout.contiguous(), lse, ctx.scale, ctx.causal)
        return dq, dk, dv, None, None


def flash_attention(q, k, v, scale=None, causal=True, return_lse=False):
    """Scaled dot-product attention of [B, H, S, hd] tensors (float32 or
    bfloat16, on the GPU), differentiable in q, k and v.  scale=None means
    1/sqrt(hd)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    out, lse = FlashAttentionFn.apply(q, k, v, float(scale), bool(causal))
    return (out, lse) if return_lse else out

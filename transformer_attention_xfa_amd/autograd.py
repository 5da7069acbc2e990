"""Autograd node over the C ABI: the differentiable attention op.

The pages' framework exposes fused attention as one op whose backward node
keeps the forward's inputs, its output and the O(S) logsumexp L next to them
(T14 flash-attention design doc, "What flash-attention is" and Key Design
Decision 2: L is what lets the backward recompute P instead of storing it).
This is that node for PyTorch: `forward` runs xfa_fwd and saves
(q, k, v, out, L); `backward` runs xfa_bwd_preprocess and xfa_bwd.  Nothing of
size S x S is kept.  Every step runs in libxfa.so; there is no fallback.

`core="fp32"` is the pages' numerics for bfloat16 tensors (same doc, the
boundary of the fused op: a bf16 call upcasts to fp32, runs the fp32 kernel
and casts the result back; L stays fp32): the casts happen at this boundary
and the attention runs in libxfa.so's fp32 kernels, so P and dS are never
rounded to bf16.  The saved tensors stay bf16 (the backward upcasts q, k, v,
the bf16 out and dO).  `core="native"` (default) runs the bf16 kernels:
bf16 operands on the matrix cores, fp32 accumulation.
"""

from __future__ import annotations

import math

import torch

from . import _binding as _b


class FlashAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, causal, fp32_core=False, dropout_p=0.0, seed=0):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        drop = dict(dropout_p=dropout_p, seed=seed)
        if fp32_core:
            out32, lse = _b.forward(q.float(), k.float(), v.float(), scale, causal, **drop)
            out = out32.to(q.dtype)
        else:
            out, lse = _b.forward(q, k, v, scale, causal, **drop)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.scale, ctx.causal, ctx.fp32_core, ctx.drop = scale, causal, fp32_core, drop
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        if ctx.fp32_core:
            dq, dk, dv = _b.backward(q.float(), k.float(), v.float(), out.float(), dout.float().contiguous(), lse,
                                     ctx.scale, ctx.causal, **ctx.drop)
            dq, dk, dv = dq.to(q.dtype), dk.to(q.dtype), dv.to(q.dtype)
        else:
            dq, dk, dv = _b.backward(q, k, v, out, dout.contiguous(), lse, ctx.scale, ctx.causal, **ctx.drop)
        return dq, dk, dv, None, None, None, None, None


CORES = ("native", "fp32")


def flash_attention(q, k, v, scale=None, causal=True, return_lse=False, core="native", dropout_p=0.0, seed=0):
    """Scaled dot-product attention of [B, H, S, hd] tensors (float32 or
    bfloat16, on the GPU), differentiable in q, k and v.  scale=None means
    1/sqrt(hd).  core: "native" runs the kernels of the tensors' dtype;
    "fp32" runs bfloat16 tensors through the fp32 kernels (casts at the
    boundary, the pages' numerics), and is the same as "native" for float32
    tensors.  dropout_p in [0, 1) drops attention probabilities with keep
    decisions drawn from (seed, element index) by a counter-based generator
    and scales the kept ones by 1/(1-p); the backward regenerates the same
    decisions.  Pass a fresh seed per step and per call site."""
    if core not in CORES:
        raise ValueError(f"core must be one of {CORES}, got {core!r}")
    if not 0.0 <= float(dropout_p) < 1.0:
        raise ValueError(f"dropout_p must be in [0, 1), got {dropout_p!r}")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    fp32_core = core == "fp32" and q.dtype == torch.bfloat16
    out, lse = FlashAttentionFn.apply(q, k, v, float(scale), bool(causal), fp32_core, float(dropout_p),
                                      int(seed) & 0xFFFFFFFFFFFFFFFF)
    return (out, lse) if return_lse else out

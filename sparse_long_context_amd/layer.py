"""Autograd wrapper of the Lighthouse Attention layer.

`lighthouse_attention(q, k, v, p, L, S)` runs lh_layer_fwd on the current
stream, keeps the buffers the forward filled, and runs lh_layer_bwd in the
backward.  The selection carries no gradient (gist.science explainer "Long
Context Pre-Training with Lighthouse Attention", technical summary 2.B).
"""
from __future__ import annotations

import torch

from . import ops


class LighthouseAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, p, L, S, out_dtype, scale, scatter_mode, sigma_mode, strata_mode):
        c = ops.Ctx(ops.make_dims(q, p, L, S, out_dtype, scale, scatter_mode, sigma_mode,
                                  strata_mode))
        o, saved = ops.layer_fwd(c, q.contiguous(), k.contiguous(), v.contiguous())
        ctx.c = c
        ctx.saved = saved
        return o

    @staticmethod
    def backward(ctx, dout):
        dq, dk, dv = ops.layer_bwd(ctx.c, ctx.saved, dout.contiguous().to(ctx.c.out))
        return dq, dk, dv, None, None, None, None, None, None, None, None


def lighthouse_attention(q, k, v, p: int, L: int, S: int, out_dtype=None, scale: float = 0.0,
                         scatter_mode: str = "hold", sigma_mode: str = "sum",
                         strata_mode: str = "joint"):
    """q, k, v: [B, H, N, d] device tensors (bf16 or float32).  Returns O
    [B, H, N, d] in out_dtype (default: the input dtype).  scatter_mode:
    "hold" (causal hold) or "span" (span broadcast); sigma_mode: how the two
    scores combine ("sum", "max" or "product"); strata_mode: one ranking
    across a stratum's levels ("joint") or a quota per level ("per_level")."""
    return LighthouseAttention.apply(q, k, v, p, L, S, out_dtype, scale, scatter_mode, sigma_mode,
                                     strata_mode)

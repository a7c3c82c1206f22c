"""Autograd binding of the causal attention calls (argument marshalling only).

A fused operation joins the autograd graph through its vector-Jacobian product
("Module and Parameter Lifecycle", "Forward and backward responsibilities": the
custom_gradient seam takes the fused output, its inputs and a callback that maps
the upstream gradient to one gradient per positional input, whose count and
shapes are validated before anything is accumulated).  Here that seam is a
torch.autograd.Function: the forward runs attn_causal_fwd and keeps Q, K, V, O
and the per-row log-sum-exp; the backward runs attn_causal_bwd on the incoming
cotangent of O and checks that each gradient has its input's shape.  Both steps
run in the HIP kernels; nothing is recomputed here.
"""
import math

import torch

from ._binding import attn_causal_bwd, attn_causal_fwd


class CausalAttentionFunction(torch.autograd.Function):
    """O = softmax(scale Q K^T, keys after the query masked) V for Q [B,Hq,T,D] and
    K, V [B,Hkv,T,D] (Hq % Hkv == 0); float32 GPU tensors."""

    @staticmethod
    def forward(ctx, q, k, v, scale):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = attn_causal_fwd(q, k, v, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_causal_bwd(q, k, v, o, lse, dout.contiguous(), scale=ctx.scale)
        for g, x in ((dq, q), (dk, k), (dv, v)):
            if g.shape != x.shape:
                raise RuntimeError(f"causal attention VJP returned {tuple(g.shape)} for an input {tuple(x.shape)}")
        return dq, dk, dv, None


def causal_attention(q, k, v, scale=None):
    """Differentiable causal attention (see CausalAttentionFunction); scale
    defaults to 1/sqrt(D)."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    return CausalAttentionFunction.apply(q, k, v, scale)

"""PyTorch autograd entry point over the C ABI (argument marshalling only).

``attention(q, k, v, causal, scale)`` returns O and records a backward that
calls ``fa2_bwd`` (or ``fa2_bwd_qk``) with the forward's O and L, so a model
can drop it in where it would call standard attention: the "FlashAttention
(v2)" glossary page calls adopting the method a choice of backend, since the
output matches standard attention exactly.  Every arithmetic step runs in the
HIP kernels; this module only makes tensors contiguous and routes them.

Shapes: q [B, H, Nq, d], k and v [B, H, Nk, d], bf16 on the GPU; causal masks
are aligned bottom-right when Nq != Nk (see ``include/fa2.h``).
"""

import torch

from . import fa2


class FlashAttention2(torch.autograd.Function):
    """O = softmax(scale q k^T, masked) v, with the tiled forward and backward kernels."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = fa2.bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal=False, scale=None):
    """Differentiable exact attention; ``scale`` defaults to 1/sqrt(d)."""
    if scale is None:
        scale = fa2.default_scale(q.shape[-1])
    return FlashAttention2.apply(q, k, v, bool(causal), float(scale))

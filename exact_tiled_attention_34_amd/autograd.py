"""PyTorch autograd entry point over the C ABI (argument marshalling only).

``attention(q, k, v, causal, scale)`` returns O and records a backward that
calls ``fa2_bwd`` (or ``fa2_bwd_qk``) with the forward's O and L, so a model
can drop it in where it would call standard attention: the "FlashAttention
(v2)" glossary page calls adopting the method a choice of backend, since the
output matches standard attention exactly.  Every arithmetic step runs in the
HIP kernels; this module only routes tensors (copying one only if its last
dimension is not contiguous).

Shapes: q [B, H, Nq, d], k and v [B, H, Nk, d], bf16 on the GPU, any strides
with a contiguous last dimension (the kernels read strided views directly);
causal masks are aligned bottom-right when Nq != Nk (see ``include/fa2.h``).
``attention_qkvpacked`` takes the fused [B, S, 3, H, d] output of a QKV
projection and returns O as [B, S, H, d]: the kernels read Q, K and V out of
the fused tensor and write O and the fused gradient in place, with no copies.
"""

import torch

from . import fa2


class FlashAttention2(torch.autograd.Function):
    """O = softmax(scale q k^T, masked) v, with the tiled forward and backward kernels."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        q, k, v = (t if t.stride(-1) == 1 else t.contiguous() for t in (q, k, v))
        o, lse = fa2.fwd(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        do = do if do.stride(-1) == 1 else do.contiguous()
        dq, dk, dv = fa2.bwd(q, k, v, o, lse, do, causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


class FlashAttention2QKVPacked(torch.autograd.Function):
    """O [B, S, H, d] from a fused qkv [B, S, 3, H, d]; the gradient is fused the same way."""

    @staticmethod
    def forward(ctx, qkv, causal, scale):
        if qkv.stride(-1) != 1:
            qkv = qkv.contiguous()
        B, S, three, H, d = qkv.shape
        q, k, v = (qkv[:, :, j].transpose(1, 2) for j in range(3))      # [B, H, S, d] views
        o = torch.empty((B, S, H, d), dtype=qkv.dtype, device=qkv.device)
        _, lse = fa2.fwd(q, k, v, causal=causal, scale=scale, out=o.transpose(1, 2))
        ctx.save_for_backward(qkv, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        qkv, o, lse = ctx.saved_tensors
        if do.stride(-1) != 1:
            do = do.contiguous()
        q, k, v = (qkv[:, :, j].transpose(1, 2) for j in range(3))
        dqkv = torch.empty_like(qkv, memory_format=torch.contiguous_format)
        dq, dk, dv = (dqkv[:, :, j].transpose(1, 2) for j in range(3))
        fa2.bwd(q, k, v, o.transpose(1, 2), lse, do.transpose(1, 2), causal=ctx.causal, scale=ctx.scale,
                dq=dq, dk=dk, dv=dv)
        return dqkv, None, None


def attention(q, k, v, causal=False, scale=None):
    """Differentiable exact attention; ``scale`` defaults to 1/sqrt(d)."""
    if scale is None:
        scale = fa2.default_scale(q.shape[-1])
    return FlashAttention2.apply(q, k, v, bool(causal), float(scale))


def attention_qkvpacked(qkv, causal=False, scale=None):
    """Differentiable exact attention over a fused qkv [B, S, 3, H, d]; returns O [B, S, H, d]."""
    if scale is None:
        scale = fa2.default_scale(qkv.shape[-1])
    return FlashAttention2QKVPacked.apply(qkv, bool(causal), float(scale))

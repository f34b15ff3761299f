"""GPT-3-2.7B-shaped self-attention sublayer with synthetic weights (a workload).

The end-to-end results on the "FlashAttention-2: Faster Attention with Better
Parallelism and Work Partitioning" page (Table 1) train GPT-3 1.3B/2.7B models
at 2k and 8k context; this module builds only the part that the attention
kernels serve, one attention sublayer of the 2.7B shape (hidden 2560, 32 heads
of 80), with caller-supplied weights and no data and no training:

    qkv = x W_qkv                    (plain library GEMM, [B*S, h] x [h, 3h])
    a = attention(qkv, causal)       (the HIP kernels, fa2_fwd / fa2_bwd, reading
                                      Q, K, V out of the fused [B, S, 3, H, d]
                                      tensor and writing a as [B, S, H, d])
    y = a W_out                      (plain library GEMM)

Backward runs through PyTorch autograd, with
``autograd.FlashAttention2QKVPacked`` calling fa2_bwd, which writes the fused
gradient of qkv directly; no tensor is copied to change its layout.  The GEMMs
are 2-D matrix products on purpose (no batched products of transposed views).

``model_flops`` applies the page's accounting for end-to-end throughput,
6 x sequence length x parameters + 12 x layers x hidden x sequence length^2
per sequence, with the attention term not halved for causal masking (as that
page says Megatron-LM and prior reports count it), here for one layer whose
parameters are the 4 hidden^2 projection weights.
"""

import torch

from .autograd import attention_qkvpacked


class AttentionBlock:
    def __init__(self, w_qkv, w_out, heads):
        hidden = w_out.shape[0]
        if w_qkv.shape != (hidden, 3 * hidden) or hidden % heads:
            raise ValueError("w_qkv must be [hidden, 3*hidden] and heads must divide hidden")
        self.w_qkv, self.w_out, self.heads = w_qkv, w_out, heads
        self.hidden, self.head_dim = hidden, hidden // heads

    def parameters(self):
        return [self.w_qkv, self.w_out]

    def __call__(self, x, causal=True):
        B, S, h = x.shape
        H, d = self.heads, self.head_dim
        qkv = torch.mm(x.reshape(B * S, h), self.w_qkv)              # [B*S, 3h]
        a = attention_qkvpacked(qkv.view(B, S, 3, H, d), causal=causal)  # [B, S, H, d]
        return torch.mm(a.view(B * S, h), self.w_out).view(B, S, h)


def model_flops(B, S, hidden, layers=1):
    """Forward + backward model FLOPs of ``layers`` attention sublayers on B sequences of S tokens."""
    params = 4 * hidden * hidden * layers
    return B * (6.0 * S * params + 12.0 * layers * hidden * S * S)

"""PyTorch integration: the fused forward and the recomputing backward as one
differentiable operation.

What it follows: FlashAttention-2 review, 'implementation requirements'
answer, section 1 (3) (a framework extension that wires the kernels' forward
and their gradient into autograd), and the call signature of the 'Flash
Attention-3' post's code example: flash_attention(query, key, value) on
[B, H, N, d] tensors with scale d^-1/2.

Only O and LSE are kept for the backward (plus the inputs), never the N x N
matrices: the backward recomputes P from LSE in the kernels.  Marshalling only;
every step runs in libattn.so.
"""
import math

import torch

from .attn import attn_bwd, attn_fwd


class FlashAttentionFn(torch.autograd.Function):
    """O = softmax(scale Q K^T [+ causal mask]) V with the kernels' backward."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = attn_fwd(q, k, v, scale=scale, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        # gradients come back in the inputs' dtype (bf16 ones are rounded once from fp32 accumulators)
        dq, dk, dv = attn_bwd(q, k, v, o, do.to(q.dtype).contiguous(), lse, scale=ctx.scale,
                              causal=ctx.causal, grad_dtype=q.dtype)
        return dq, dk, dv, None, None


def flash_attention(query, key, value, scale=None, causal=False):
    """Exact attention over [B, H, N, d] tensors (fp32 or bf16, on a GPU), differentiable.

    scale defaults to 1/sqrt(d); causal masks keys after each query.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(query.shape[-1])
    return FlashAttentionFn.apply(query, key, value, float(scale), bool(causal))

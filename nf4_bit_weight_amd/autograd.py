"""Checkpoint-visible autograd wrappers over the fused NF4 kernels.

Soup issue #842 ("Layer streaming: a checkpoint-visible fused NF4
dequantise-and-multiply"), "Design sketch": save only through
save_for_backward -- the packed nibbles, the absmax and the nested statistics
-- and hold no tensor on ctx as an attribute; the backward computes only
grad_x = grad_y @ W with the transposed fused kernel and never materialises a
dense W.  bitsandbytes issue #2034, "Root cause" / "Why save_for_backward
fixes it", explains why: torch.utils.checkpoint re-materialises only what went
through save_for_backward, and the saved tensors carry autograd's version
counter, so an in-place change of a saved weight between forward and backward
raises instead of silently producing wrong gradients.

Only integers (N, K, E) and the caller's dtype live on ctx.  The weight is
frozen: no gradient is returned for any weight field.

dtype handling follows Linear4bit's forward (Soup issue #842, "Design
sketch": the Function keeps its dtype behaviour): the kernels compute in bf16
with fp32 accumulation, and the output (and the input gradient) come back in
the dtype the caller passed in.
"""

from __future__ import annotations

import torch

from . import api
from .api import NF4Weight


def _weight(saved, N, K, bits) -> NF4Weight:
    packed, absmax, nabs, noff, code, ncode = saved
    return NF4Weight(packed, absmax, nabs, noff, code, ncode, N, K, bits)


class NF4MatMul(torch.autograd.Function):
    """y = x . W_hat^T with W given as its NF4 fields (frozen)."""

    @staticmethod
    def forward(ctx, x, packed, absmax, nested_absmax, nested_offset, code, nested_code, N, K, bits=4):
        w = NF4Weight(packed, absmax, nested_absmax, nested_offset, code, nested_code, N, K, bits)
        lead = x.shape[:-1]
        x2 = x.reshape(-1, K)
        if x2.dtype != torch.bfloat16:
            x2 = x2.to(torch.bfloat16)
        y = api.nf4_matmul_fwd(x2.contiguous(), w)
        ctx.save_for_backward(packed, absmax, nested_absmax, nested_offset, code, nested_code)
        ctx.N, ctx.K, ctx.bits = int(N), int(K), int(bits)
        ctx.x_dtype = x.dtype
        return y.reshape(*lead, N).to(x.dtype)

    @staticmethod
    def backward(ctx, grad_y):
        w = _weight(ctx.saved_tensors, ctx.N, ctx.K, ctx.bits)
        grad_x = None
        if ctx.needs_input_grad[0]:
            lead = grad_y.shape[:-1]
            g2 = grad_y.reshape(-1, ctx.N)
            if g2.dtype != torch.bfloat16:
                g2 = g2.to(torch.bfloat16)
            grad_x = api.nf4_matmul_bwd_input(g2.contiguous(), w).reshape(*lead, ctx.K)
            grad_x = grad_x.to(ctx.x_dtype)
        return grad_x, None, None, None, None, None, None, None, None, None


class NF4GroupedMatMul(torch.autograd.Function):
    """Per-expert y over expert-sorted rows (Experts PR, "Commit 2": a frozen
    expert projection whose backward is grad_output @ W on the expert slice)."""

    @staticmethod
    def forward(ctx, x, offsets, packed, absmax, nested_absmax, nested_offset, code, nested_code,
                E, N, K, bits=4):
        w = NF4Weight(packed, absmax, nested_absmax, nested_offset, code, nested_code, N, K, bits)
        x2 = x if x.dtype == torch.bfloat16 else x.to(torch.bfloat16)
        y = api.nf4_grouped_matmul_fwd(x2.contiguous(), offsets, w, E)
        ctx.save_for_backward(offsets, packed, absmax, nested_absmax, nested_offset, code,
                              nested_code)
        ctx.E, ctx.N, ctx.K, ctx.bits = int(E), int(N), int(K), int(bits)
        ctx.x_dtype = x.dtype
        return y.to(x.dtype)

    @staticmethod
    def backward(ctx, grad_y):
        offsets, *rest = ctx.saved_tensors
        w = _weight(rest, ctx.N, ctx.K, ctx.bits)
        grad_x = None
        if ctx.needs_input_grad[0]:
            g = grad_y if grad_y.dtype == torch.bfloat16 else grad_y.to(torch.bfloat16)
            grad_x = api.nf4_grouped_matmul_bwd_input(g.contiguous(), offsets, w, ctx.E)
            grad_x = grad_x.to(ctx.x_dtype)
        return (grad_x,) + (None,) * 11


def nf4_linear(x: torch.Tensor, w: NF4Weight) -> torch.Tensor:
    """F.linear(x, W_hat) for a frozen NF4 weight, differentiable in x."""
    return NF4MatMul.apply(x, *w.tensors(), w.N, w.K, w.bits)


def nf4_grouped_linear(x: torch.Tensor, offsets: torch.Tensor, w: NF4Weight, E: int) -> torch.Tensor:
    return NF4GroupedMatMul.apply(x, offsets, *w.tensors(), E, w.N, w.K, w.bits)

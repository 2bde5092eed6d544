"""Autograd wrapper: fused linear cross-entropy as a differentiable torch op.

The forward runs ``flce_fwd`` (loss and the per-token LSE, no logits kept);
the backward runs ``flce_bwd``, which recomputes the logits chunk by chunk
and forms the gradient from the saved LSE -- the split of the blog page
"Liger Kernel: Fused Triton Kernels for LLM Training", section "2. In-Kernel
Gradient Computation During the Backward Pass".  The upstream gradient of the
loss is handed to the kernels as a device scalar.  Call shape as the fused
loss module on the lecture page: ``loss_fn(hidden [B*S, D], weight [V, D],
labels [B*S])``.  ``CrossEntropyLoss`` does the same for logits that are
already materialised.
"""
from __future__ import annotations

import torch

from . import cross_entropy, cross_entropy_backward, linear_cross_entropy_backward, linear_cross_entropy_forward


class LinearCrossEntropyFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, labels, ignore_index: int = -100, reduction: str = "mean"):
        loss, lse = linear_cross_entropy_forward(hidden, weight, labels, ignore_index, reduction)
        ctx.save_for_backward(hidden, weight, labels, lse)
        ctx.ignore_index = ignore_index
        ctx.reduction = reduction
        return loss.view(())

    @staticmethod
    def backward(ctx, grad_loss):
        hidden, weight, labels, lse = ctx.saved_tensors
        g = grad_loss.reshape(1)
        if g.dtype != torch.float32 or not g.is_contiguous():
            g = g.to(torch.float32).contiguous()
        dh, dw = linear_cross_entropy_backward(hidden, weight, labels, lse, g, ctx.ignore_index, ctx.reduction)
        return dh, dw, None, None, None


def linear_cross_entropy_loss(hidden, weight, labels, ignore_index: int = -100, reduction: str = "mean"):
    return LinearCrossEntropyFunction.apply(hidden, weight, labels, ignore_index, reduction)


class LinearCrossEntropyLoss(torch.nn.Module):
    """Cross-entropy of softmax(hidden . weight^T) against labels without materialising the logits."""

    def __init__(self, ignore_index: int = -100, reduction: str = "mean"):
        super().__init__()
        if reduction not in ("mean", "sum"):
            raise ValueError(f"unknown reduction {reduction!r}")
        self.ignore_index = ignore_index
        self.reduction = reduction

    def forward(self, hidden, weight, labels):
        return LinearCrossEntropyFunction.apply(hidden, weight, labels, self.ignore_index, self.reduction)


class CrossEntropyFunction(torch.autograd.Function):
    """Cross-entropy on given logits: loss and LSE in the forward, the gradient from
    the saved LSE in the backward (one read and one write of the logits)."""

    @staticmethod
    def forward(ctx, logits, labels, ignore_index: int = -100, reduction: str = "mean"):
        loss, lse, _ = cross_entropy(logits, labels, ignore_index, reduction, grad=None)
        ctx.save_for_backward(logits, labels, lse)
        ctx.ignore_index = ignore_index
        ctx.reduction = reduction
        return loss.view(())

    @staticmethod
    def backward(ctx, grad_loss):
        logits, labels, lse = ctx.saved_tensors
        g = grad_loss.reshape(1)
        if g.dtype != torch.float32 or not g.is_contiguous():
            g = g.to(torch.float32).contiguous()
        grad = cross_entropy_backward(logits, labels, lse, g, ctx.ignore_index, ctx.reduction)
        return grad, None, None, None


class CrossEntropyLoss(torch.nn.Module):
    """Cross-entropy of softmax(logits) against labels, call shape ``loss_fn(logits [N, V], labels [N])``."""

    def __init__(self, ignore_index: int = -100, reduction: str = "mean"):
        super().__init__()
        if reduction not in ("mean", "sum"):
            raise ValueError(f"unknown reduction {reduction!r}")
        self.ignore_index = ignore_index
        self.reduction = reduction

    def forward(self, logits, labels):
        return CrossEntropyFunction.apply(logits, labels, self.ignore_index, self.reduction)

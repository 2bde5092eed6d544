"""Autograd wrapper: fused linear cross-entropy as a differentiable torch op.

By default the forward runs ``flce_fwd`` (loss and the per-token LSE, no
logits kept) and the backward runs ``flce_bwd``, which recomputes the logits
chunk by chunk and forms the gradient from the saved LSE -- the split of the
blog page "Liger Kernel: Fused Triton Kernels for LLM Training", section "2.
In-Kernel Gradient Computation During the Backward Pass" (8 N D V flop).
With ``one_pass=True`` the forward runs ``flce_fwd_bwd`` instead, which forms
dH and dW from the chunk's logits in the same pass as the loss (6 N D V
flop, as in the blog's simulation of the method) and keeps them until the
backward scales them by the upstream gradient (``flce_scale``); that holds
[N, D] + [V, D] gradient bytes between forward and backward, and the graph
allows one backward.  The upstream gradient reaches the kernels as a device
scalar either way.  Call shape as the fused loss module on the lecture page:
``loss_fn(hidden [B*S, D], weight [V, D], labels [B*S])``.
``CrossEntropyLoss`` does the same for logits that are already materialised.
"""
from __future__ import annotations

import torch

from . import (cross_entropy, cross_entropy_backward, linear_cross_entropy, linear_cross_entropy_backward,
               linear_cross_entropy_forward, scale_)


def _upstream(grad_loss):
    g = grad_loss.reshape(1)
    if g.dtype != torch.float32 or not g.is_contiguous():
        g = g.to(torch.float32).contiguous()
    return g


class LinearCrossEntropyFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, labels, ignore_index: int = -100, reduction: str = "mean",
                one_pass: bool = False):
        ctx.ignore_index = ignore_index
        ctx.reduction = reduction
        ctx.one_pass = bool(one_pass) and (ctx.needs_input_grad[0] or ctx.needs_input_grad[1])
        if ctx.one_pass:
            loss, _, dh, dw = linear_cross_entropy(hidden, weight, labels, ignore_index, reduction)
            ctx.save_for_backward(dh, dw)
            ctx.used = False
        else:
            loss, lse = linear_cross_entropy_forward(hidden, weight, labels, ignore_index, reduction)
            ctx.save_for_backward(hidden, weight, labels, lse)
        return loss.view(())

    @staticmethod
    def backward(ctx, grad_loss):
        g = _upstream(grad_loss)
        if ctx.one_pass:
            if ctx.used:
                raise RuntimeError("a one_pass linear cross-entropy graph allows one backward: its saved "
                                   "gradients are scaled in place")
            ctx.used = True
            dh, dw = ctx.saved_tensors
            scale_(dh, g)
            scale_(dw, g)
        else:
            hidden, weight, labels, lse = ctx.saved_tensors
            dh, dw = linear_cross_entropy_backward(hidden, weight, labels, lse, g, ctx.ignore_index, ctx.reduction)
        return (dh if ctx.needs_input_grad[0] else None, dw if ctx.needs_input_grad[1] else None,
                None, None, None, None)


def linear_cross_entropy_loss(hidden, weight, labels, ignore_index: int = -100, reduction: str = "mean",
                              one_pass: bool = False):
    return LinearCrossEntropyFunction.apply(hidden, weight, labels, ignore_index, reduction, one_pass)


class LinearCrossEntropyLoss(torch.nn.Module):
    """Cross-entropy of softmax(hidden . weight^T) against labels without materialising the logits.

    ``one_pass=True`` computes dH and dW in the forward (flce_fwd_bwd) and keeps them
    for the backward: 6 N D V flop instead of 8, for [N, D] + [V, D] gradient bytes
    held between the two and a graph that allows one backward.
    """

    def __init__(self, ignore_index: int = -100, reduction: str = "mean", one_pass: bool = False):
        super().__init__()
        if reduction not in ("mean", "sum"):
            raise ValueError(f"unknown reduction {reduction!r}")
        self.ignore_index = ignore_index
        self.reduction = reduction
        self.one_pass = one_pass

    def forward(self, hidden, weight, labels):
        return LinearCrossEntropyFunction.apply(hidden, weight, labels, self.ignore_index, self.reduction,
                                                self.one_pass)


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
        g = _upstream(grad_loss)
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

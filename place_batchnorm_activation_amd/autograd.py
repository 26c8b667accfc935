"""PyTorch autograd binding of the In-Place ABN library.

`InPlaceABN` is a drop-in replacement for `BatchNorm2d` followed by an invertible
activation (leaky ReLU, ELU or identity).  The forward writes y over its input
(the input must not be needed by any other autograd node, e.g. a convolution's
output), and autograd keeps only y and three per-channel vectors for the
backward, which rebuilds what it needs from y (section 3 of the paperlayer
summary of "In-Place Activated BatchNorm for Memory-Optimized Training of DNNs",
"INPLACE-ABN").  Every computation runs in the library's HIP kernels through the
C ABI; this module only marshals tensors and streams.

Layout follows the tensor's memory format: contiguous tensors are NCHW,
channels_last tensors NHWC.  Storage dtypes: float32, bfloat16, float16; the
affine parameters and statistics are float32.
"""
from __future__ import annotations

import torch

from . import (iabn_backward, iabn_backward_eval, iabn_forward_eval, iabn_forward_train,
               workspace)


def _layout(x: torch.Tensor) -> str:
    if x.dim() != 4:
        raise ValueError("InPlaceABN expects a 4-d tensor [N, C, H, W], got %d-d" % x.dim())
    if x.is_contiguous():
        return "NCHW"
    if x.is_contiguous(memory_format=torch.channels_last):
        return "NHWC"
    raise ValueError("InPlaceABN needs a contiguous or channels_last tensor")


def _like(t: torch.Tensor, layout: str) -> torch.Tensor:
    """t in the memory format of `layout` (a copy only when it differs)."""
    fmt = torch.channels_last if layout == "NHWC" else torch.contiguous_format
    return t.contiguous(memory_format=fmt)


class InPlaceABNFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, running_mean, running_var, training, momentum, eps,
                activation, act_param):
        layout = _layout(x)
        N, C, H, W = x.shape
        ws = workspace(N, C, H, W, layout, x.dtype, x.device)
        if training:
            save_mean = torch.empty(C, device=x.device, dtype=torch.float32)
            save_invstd = torch.empty(C, device=x.device, dtype=torch.float32)
            iabn_forward_train(x, N, C, H, W, layout, weight, bias, running_mean, running_var,
                               save_mean, save_invstd, activation, act_param, eps, momentum, ws)
            stat = save_invstd
        else:
            iabn_forward_eval(x, N, C, H, W, layout, weight, bias, running_mean, running_var,
                              activation, act_param, eps)
            stat = running_var
        ctx.mark_dirty(x)
        ctx.save_for_backward(x, weight, bias, stat)
        ctx.cfg = (training, eps, activation, act_param, layout)
        return x

    @staticmethod
    def backward(ctx, dy):
        y, weight, bias, stat = ctx.saved_tensors
        training, eps, activation, act_param, layout = ctx.cfg
        N, C, H, W = y.shape
        dy = _like(dy, layout)
        dx = torch.empty_like(dy)
        dgamma = torch.empty(C, device=y.device, dtype=torch.float32)
        dbeta = torch.empty(C, device=y.device, dtype=torch.float32)
        ws = workspace(N, C, H, W, layout, y.dtype, y.device)
        if training:
            iabn_backward(y, dy, dx, N, C, H, W, layout, weight, bias, stat, dgamma, dbeta,
                          activation, act_param, ws)
        else:
            iabn_backward_eval(y, dy, dx, N, C, H, W, layout, weight, bias, stat, eps, dgamma,
                               dbeta, activation, act_param, ws)
        return dx, dgamma, dbeta, None, None, None, None, None, None, None


class InPlaceABN(torch.nn.Module):
    """BatchNorm2d + invertible activation, computed in place.

    activation: "leaky_relu" (act_param = negative slope, > 0), "elu" (act_param =
    alpha, > 0) or "identity".  Running statistics follow BatchNorm2d's update
    (momentum, unbiased running variance).  The affine weight must stay non-zero:
    the backward divides by it when it rebuilds the normalised input."""

    def __init__(self, num_features: int, eps: float = 1e-5, momentum: float = 0.1,
                 activation: str = "leaky_relu", act_param: float = 0.01,
                 device=None):
        super().__init__()
        self.num_features = num_features
        self.eps = eps
        self.momentum = momentum
        self.activation = activation
        self.act_param = act_param
        f32 = dict(device=device, dtype=torch.float32)
        self.weight = torch.nn.Parameter(torch.ones(num_features, **f32))
        self.bias = torch.nn.Parameter(torch.zeros(num_features, **f32))
        self.register_buffer("running_mean", torch.zeros(num_features, **f32))
        self.register_buffer("running_var", torch.ones(num_features, **f32))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return InPlaceABNFunction.apply(x, self.weight, self.bias, self.running_mean,
                                        self.running_var, self.training, self.momentum, self.eps,
                                        self.activation, self.act_param)

    def extra_repr(self) -> str:
        return "%d, eps=%g, momentum=%g, activation=%s, act_param=%g" % (
            self.num_features, self.eps, self.momentum, self.activation, self.act_param)

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
channels_last (and channels_last_3d) tensors NHWC.  Any tensor [N, C, *] is
taken, as BatchNorm1d, 2d and 3d take them: the spatial extent is folded into
the library's H*W.  Storage dtypes: float32, bfloat16, float16; the
affine parameters and statistics are float32.
"""
from __future__ import annotations

import torch

from . import (iabn_backward, iabn_backward_eval, iabn_forward_eval, iabn_forward_train,
               workspace)


def _geometry(x: torch.Tensor):
    """(N, C, H, W, layout) under which the library sees x, a tensor [N, C, *]:
    contiguous tensors are NCHW with the spatial extent folded into H*W (2-d
    [N, C] and 3-d [N, C, L] tensors, as BatchNorm1d takes them, and 5-d
    [N, C, D, H, W] ones, as BatchNorm3d does), channels_last and
    channels_last_3d ones NHWC (depth folded into H)."""
    if x.dim() < 2:
        raise ValueError("InPlaceABN expects a tensor [N, C, ...], got %d-d" % x.dim())
    N, C = int(x.shape[0]), int(x.shape[1])
    sp = [int(v) for v in x.shape[2:]]
    if x.dim() == 4 and x.is_contiguous():
        return N, C, sp[0], sp[1], "NCHW"
    if x.is_contiguous():
        hw = 1
        for v in sp:
            hw *= v
        return N, C, hw, 1, "NCHW"
    if x.dim() == 4 and x.is_contiguous(memory_format=torch.channels_last):
        return N, C, sp[0], sp[1], "NHWC"
    if x.dim() == 5 and x.is_contiguous(memory_format=torch.channels_last_3d):
        return N, C, sp[0] * sp[1], sp[2], "NHWC"
    raise ValueError("InPlaceABN needs a contiguous, channels_last or channels_last_3d tensor")


def _like(t: torch.Tensor, layout: str) -> torch.Tensor:
    """t in the memory format the library reads for `layout` (a copy only when
    it differs)."""
    if layout == "NCHW":
        return t.contiguous()
    fmt = torch.channels_last if t.dim() == 4 else torch.channels_last_3d
    return t.contiguous(memory_format=fmt)


def _check_params(x, *vecs) -> None:
    """The library reads the affine parameters and statistics as float32 on x's
    device, C of each."""
    C = x.shape[1]
    for v in vecs:
        if v is None:
            continue
        if v.dtype != torch.float32 or v.device != x.device or v.numel() != C or \
                not v.is_contiguous():
            raise TypeError("InPlaceABN keeps weight, bias and running statistics as "
                            "contiguous float32 vectors of %d elements on %s; got %s %s on %s"
                            % (C, x.device, v.dtype, tuple(v.shape), v.device))


class InPlaceABNFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, running_mean, running_var, training, momentum, eps,
                activation, act_param):
        N, C, H, W, layout = _geometry(x)
        _check_params(x, weight, bias, running_mean, running_var)
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
        ctx.cfg = (training, eps, activation, act_param, (N, C, H, W, layout))
        return x

    @staticmethod
    def backward(ctx, dy):
        y, weight, bias, stat = ctx.saved_tensors
        training, eps, activation, act_param, (N, C, H, W, layout) = ctx.cfg
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
    """BatchNorm (1d, 2d or 3d: any input [N, C, *]) + invertible activation,
    computed in place.

    activation: "leaky_relu" (act_param = negative slope, > 0), "elu" (act_param =
    alpha, > 0) or "identity".  Running statistics follow BatchNorm2d's update
    (momentum, unbiased running variance; momentum=None takes the cumulative
    average over the steps so far).  affine=False fixes weight 1 and bias 0;
    track_running_stats=False keeps no running statistics and normalises with
    the batch's own in eval mode too, as BatchNorm2d does.  The affine weight
    must stay non-zero: the backward divides by it when it rebuilds the
    normalised input."""

    def __init__(self, num_features: int, eps: float = 1e-5, momentum: float = 0.1,
                 activation: str = "leaky_relu", act_param: float = 0.01,
                 device=None, affine: bool = True, track_running_stats: bool = True):
        super().__init__()
        self.num_features = num_features
        self.eps = eps
        self.momentum = momentum
        self.activation = activation
        self.act_param = act_param
        self.affine = affine
        self.track_running_stats = track_running_stats
        f32 = dict(device=device, dtype=torch.float32)
        if affine:
            self.weight = torch.nn.Parameter(torch.ones(num_features, **f32))
            self.bias = torch.nn.Parameter(torch.zeros(num_features, **f32))
        else:
            # fixed, and kept out of the state dict as BatchNorm2d keeps none
            self.register_buffer("weight", torch.ones(num_features, **f32), persistent=False)
            self.register_buffer("bias", torch.zeros(num_features, **f32), persistent=False)
        if track_running_stats:
            self.register_buffer("running_mean", torch.zeros(num_features, **f32))
            self.register_buffer("running_var", torch.ones(num_features, **f32))
            self.register_buffer("num_batches_tracked",
                                 torch.tensor(0, dtype=torch.long, device=device))
        else:
            self.running_mean = self.running_var = self.num_batches_tracked = None
        self._steps = 0                  # host copy of num_batches_tracked

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        batch_stats = self.training or not self.track_running_stats
        factor = 0.0 if self.momentum is None else self.momentum
        if self.training and self.track_running_stats:
            self._steps += 1
            self.num_batches_tracked.add_(1)
            if self.momentum is None:
                factor = 1.0 / self._steps
        return InPlaceABNFunction.apply(x, self.weight, self.bias, self.running_mean,
                                        self.running_var, batch_stats, factor, self.eps,
                                        self.activation, self.act_param)

    def _load_from_state_dict(self, state_dict, prefix, *args, **kwargs):
        super()._load_from_state_dict(state_dict, prefix, *args, **kwargs)
        if self.track_running_stats:
            self._steps = int(self.num_batches_tracked.item())

    def extra_repr(self) -> str:
        return "%d, eps=%g, momentum=%s, activation=%s, act_param=%g, affine=%s, " \
               "track_running_stats=%s" % (self.num_features, self.eps, self.momentum,
                                          self.activation, self.act_param, self.affine,
                                          self.track_running_stats)

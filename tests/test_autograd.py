"""The PyTorch autograd binding (place_batchnorm_activation_amd.autograd) on the GPU.

The binding only marshals tensors, so its outputs must be bit-identical to the
C-ABI calls that the parity tests check against the oracle; channels_last input
takes the NHWC kernels; eval mode takes the frozen-statistics pair; and the
autograd graph keeps y alone per layer (the memory claim of section 3 of the
paperlayer summary, "INPLACE-ABN").
"""
import numpy as np
import pytest
import torch

import harness
import workloads

iabn = pytest.importorskip("place_batchnorm_activation_amd")
from place_batchnorm_activation_amd.autograd import InPlaceABN  # noqa: E402

pytestmark = pytest.mark.gpu


def _module(wl, inp):
    m = InPlaceABN(wl.C, eps=wl.eps, momentum=wl.momentum, activation=wl.act,
                   act_param=wl.act_param, device="cuda")
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(inp.gamma))
        m.bias.copy_(torch.from_numpy(inp.beta))
        m.running_mean.copy_(torch.from_numpy(inp.running_mean))
        m.running_var.copy_(torch.from_numpy(inp.running_var))
    return m


CASES = [workloads.config(2).with_shape(4, 16, 12, 12),
         workloads.config(4).with_shape(3, 8, 10, 10),
         workloads.config(3).with_shape(2, 32, 8, 8),
         workloads.config(5).with_shape(8, 256, 7, 7)]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_training_matches_the_c_abi_bitwise(wl):
    inp = workloads.make_inputs(wl)
    ref = harness.run_gpu(inp)
    m = _module(wl, inp)
    x_leaf = harness.to_device(inp.x, wl).requires_grad_()
    if wl.layout == "NHWC":
        # storage is [N, H, W, C]; the module takes logical NCHW in channels_last
        x = x_leaf.permute(0, 3, 1, 2).clone(memory_format=torch.channels_last)
    else:
        x = x_leaf.clone()                   # not a leaf: the layer may write over it
    y = m(x)
    dy = harness.to_device(inp.dy, wl)
    if wl.layout == "NHWC":
        dy = dy.permute(0, 3, 1, 2)
    y.backward(dy)
    torch.cuda.synchronize()
    y_st = y.permute(0, 2, 3, 1) if wl.layout == "NHWC" else y
    assert torch.equal(y_st, ref.y)
    assert torch.equal(x_leaf.grad, ref.dx)
    assert np.array_equal(m.weight.grad.cpu().numpy(), ref.dgamma)
    assert np.array_equal(m.bias.grad.cpu().numpy(), ref.dbeta)
    assert np.array_equal(m.running_mean.cpu().numpy(), ref.running_mean)
    assert np.array_equal(m.running_var.cpu().numpy(), ref.running_var)


def test_eval_mode_uses_frozen_statistics():
    wl = workloads.config(2).with_shape(2, 8, 6, 6)
    inp = workloads.make_inputs(wl)
    m = _module(wl, inp).eval()
    rng = np.random.default_rng(3)
    with torch.no_grad():
        m.running_mean.copy_(torch.from_numpy(rng.normal(0, 1, wl.C).astype(np.float32)))
        m.running_var.copy_(torch.from_numpy(rng.uniform(0.5, 2, wl.C).astype(np.float32)))
    rm0, rv0 = m.running_mean.clone(), m.running_var.clone()
    x_leaf = harness.to_device(inp.x, wl).requires_grad_()
    y = m(x_leaf.clone())
    dy = harness.to_device(inp.dy, wl)
    y.backward(dy)
    # the same through the C ABI
    C = wl.C
    y2 = harness.to_device(inp.x, wl)
    iabn.iabn_forward_eval(y2, wl.N, C, wl.H, wl.W, "NCHW", m.weight.detach(), m.bias.detach(),
                           rm0, rv0, wl.act, wl.act_param, wl.eps)
    dx2 = torch.empty_like(dy)
    dg2, db2 = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(wl.N, C, wl.H, wl.W, "NCHW", y2.dtype)
    iabn.iabn_backward_eval(y2, dy, dx2, wl.N, C, wl.H, wl.W, "NCHW", m.weight.detach(),
                            m.bias.detach(), rv0, wl.eps, dg2, db2, wl.act, wl.act_param, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(x_leaf.grad, dx2)
    assert torch.equal(m.weight.grad, dg2) and torch.equal(m.bias.grad, db2)
    assert torch.equal(m.running_mean, rm0) and torch.equal(m.running_var, rv0)


def test_chain_keeps_one_buffer_per_layer():
    """A chain of L (1x1 convolution -> normalisation + activation) layers.  The
    conventional block keeps, per layer, the convolution output (batch norm's
    input) and the batch norm output (the activation's input) besides the
    activation output that the next convolution keeps; InPlace-ABN keeps the one
    buffer y, which is also the next convolution's input.  The saved activations
    must shrink by two tensors per layer."""
    torch.manual_seed(0)
    N, C, H, W, L = 8, 64, 32, 32, 4
    S = N * C * H * W * 4
    convs = [torch.nn.Conv2d(C, C, 1, bias=False).cuda() for _ in range(L)]

    def peak(norms):
        x = torch.randn(N, C, H, W, device="cuda", requires_grad=True)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        h = x
        for conv, norm in zip(convs, norms):
            h = norm(conv(h))
        saved = torch.cuda.memory_allocated() - base
        h.sum().backward()
        torch.cuda.synchronize()
        return saved, torch.cuda.max_memory_allocated() - base

    std = [torch.nn.Sequential(torch.nn.BatchNorm2d(C), torch.nn.LeakyReLU(0.01)).cuda()
           for _ in range(L)]
    abn = [InPlaceABN(C, device="cuda") for _ in range(L)]
    saved_std, peak_std = peak(std)
    saved_abn, peak_abn = peak(abn)
    print("saved MB: standard %.1f, in-place %.1f; peak MB: %.1f, %.1f" %
          (saved_std / 2**20, saved_abn / 2**20, peak_std / 2**20, peak_abn / 2**20))
    assert saved_std - saved_abn >= (2 * L - 0.5) * S
    assert peak_abn < peak_std

"""The PyTorch autograd binding (place_batchnorm_activation_amd.autograd) on the GPU.

The binding only marshals tensors, so its outputs must be bit-identical to the
C-ABI calls, and within the parity gates of the fp64 oracle (training and eval
mode, checked here against the oracle directly); channels_last input
takes the NHWC kernels; eval mode takes the frozen-statistics pair; and the
autograd graph keeps y alone per layer (the memory claim of section 3 of the
paperlayer summary, "INPLACE-ABN").
"""
import numpy as np
import pytest
import torch

import harness
import oracle
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


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_training_matches_the_oracle(wl):
    """The module's y, running statistics, dx, dgamma and dbeta against the fp64
    oracle: the forward on the same x bits; the backward on the module's own y
    bits, with the oracle's invstd (the module keeps save_invstd to itself; the
    two agree to fp32 rounding, far inside the gates)."""
    inp = workloads.make_inputs(wl)
    m = _module(wl, inp)
    x_leaf = harness.to_device(inp.x, wl).requires_grad_()
    x = (x_leaf.permute(0, 3, 1, 2).clone(memory_format=torch.channels_last)
         if wl.layout == "NHWC" else x_leaf.clone())
    y = m(x)
    dy = harness.to_device(inp.dy, wl)
    y.backward(dy.permute(0, 3, 1, 2) if wl.layout == "NHWC" else dy)
    torch.cuda.synchronize()
    y_st = y.detach().permute(0, 2, 3, 1) if wl.layout == "NHWC" else y.detach()
    a = harness.f32(wl.act_param)
    xo = harness.storage_channels(inp.x, wl)
    f = oracle.forward_train(xo, inp.gamma, inp.beta, wl.act, a, harness.f32(wl.eps),
                             harness.f32(wl.momentum), inp.running_mean, inp.running_var,
                             storage=wl.dtype)
    yg = harness.to_nchw64(y_st, wl)
    o = oracle.backward_from_y(yg, harness.storage_channels(inp.dy, wl), inp.gamma, inp.beta,
                               f["invstd"], wl.act, a)
    err = {"y": harness.rel_err_tensor(yg, f["y"]),
           "running_mean": harness.rel_err_vec(m.running_mean.cpu().numpy(), f["running_mean"]),
           "running_var": harness.rel_err_vec(m.running_var.cpu().numpy(), f["running_var"]),
           "dx": harness.rel_err_tensor(harness.to_nchw64(x_leaf.grad, wl), o["dx"]),
           "dgamma": harness.rel_err_vec(m.weight.grad.cpu().numpy(), o["dgamma"]),
           "dbeta": harness.rel_err_vec(m.bias.grad.cpu().numpy(), o["dbeta"])}
    print("case:", wl.name, err, flush=True)
    harness.assert_within(err, wl.dtype, wl.name)


def test_eval_mode_matches_the_oracle():
    """Eval mode (frozen running statistics) against the oracle's inference forward
    and its backward with the statistics frozen."""
    wl = workloads.config(4).with_shape(3, 8, 10, 10)
    inp = workloads.make_inputs(wl)
    m = _module(wl, inp).eval()
    rng = np.random.default_rng(5)
    rm = rng.normal(0, 1, wl.C).astype(np.float32)
    rv = rng.uniform(0.5, 2, wl.C).astype(np.float32)
    with torch.no_grad():
        m.running_mean.copy_(torch.from_numpy(rm))
        m.running_var.copy_(torch.from_numpy(rv))
    x_leaf = harness.to_device(inp.x, wl).requires_grad_()
    y = m(x_leaf.clone())
    dy = harness.to_device(inp.dy, wl)
    y.backward(dy)
    torch.cuda.synchronize()
    a, eps = harness.f32(wl.act_param), harness.f32(wl.eps)
    yo = oracle.forward_eval(harness.storage_channels(inp.x, wl), inp.gamma, inp.beta, rm, rv,
                             wl.act, a, eps, storage=wl.dtype)
    yg = harness.to_nchw64(y.detach(), wl)
    o = oracle.backward_eval(yg, harness.storage_channels(inp.dy, wl), inp.gamma, inp.beta, rv,
                             wl.act, a, eps)
    err = {"y": harness.rel_err_tensor(yg, yo),
           "dx": harness.rel_err_tensor(harness.to_nchw64(x_leaf.grad, wl), o["dx"]),
           "dgamma": harness.rel_err_vec(m.weight.grad.cpu().numpy(), o["dgamma"]),
           "dbeta": harness.rel_err_vec(m.bias.grad.cpu().numpy(), o["dbeta"])}
    print("eval:", err, flush=True)
    harness.assert_within(err, wl.dtype, "eval")


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


def _run_module(x_in, C, dy_in, seed=0):
    """One training step of a fresh module on x_in (not a leaf): y, dx, dgamma,
    dbeta, running statistics."""
    torch.manual_seed(seed)
    m = InPlaceABN(C, device="cuda")
    with torch.no_grad():
        m.weight.copy_(torch.rand(C) + 0.5)
        m.bias.copy_(0.1 * torch.randn(C))
    leaf = x_in.detach().clone().requires_grad_()
    x = leaf.clone(memory_format=torch.preserve_format)
    y = m(x)
    y.backward(dy_in)
    torch.cuda.synchronize()
    return (y.detach(), leaf.grad, m.weight.grad, m.bias.grad, m.running_mean.clone(),
            m.running_var.clone())


@pytest.mark.parametrize("shape,fmt", [((64, 96), None), ((8, 32, 300), None),
                                       ((2, 16, 6, 10, 12), None),
                                       ((2, 16, 6, 10, 12), torch.channels_last_3d),
                                       ((4, 64, 5, 7, 9), torch.channels_last_3d)],
                         ids=["1d_NC", "1d_NCL", "3d", "3d_channels_last", "3d_cl_64ch"])
def test_any_batchnorm_input_matches_its_4d_form(shape, fmt):
    """BatchNorm1d / 3d inputs: the bits of the same step on the 4-d tensor the
    library sees (spatial extent folded into H*W; depth into H when channels
    last)."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(shape, generator=g).cuda()
    dy = torch.randn(shape, generator=g).cuda()
    N, C = shape[:2]
    if fmt is None:
        x4 = x.reshape(N, C, -1, 1)
        dy4 = dy.reshape(N, C, -1, 1)
    else:
        x = x.contiguous(memory_format=fmt)
        dy = dy.contiguous(memory_format=fmt)
        D, H, W = shape[2:]
        # [N, D, H, W, C] memory -> [N, D*H, W, C] -> logical NCHW in channels_last
        x4 = x.permute(0, 2, 3, 4, 1).reshape(N, D * H, W, C).permute(0, 3, 1, 2)
        dy4 = dy.permute(0, 2, 3, 4, 1).reshape(N, D * H, W, C).permute(0, 3, 1, 2)
        assert x4.is_contiguous(memory_format=torch.channels_last)
    a = _run_module(x, C, dy)
    b = _run_module(x4, C, dy4)
    assert torch.equal(a[0].reshape(-1) if fmt is None else a[0].permute(0, 2, 3, 4, 1).reshape(-1),
                       b[0].reshape(-1) if fmt is None else b[0].permute(0, 2, 3, 1).reshape(-1))
    assert torch.equal(a[1].reshape(b[1].shape) if fmt is None else
                       a[1].permute(0, 2, 3, 4, 1).reshape(-1),
                       b[1] if fmt is None else b[1].permute(0, 2, 3, 1).reshape(-1))
    for u, v in zip(a[2:], b[2:]):
        assert torch.equal(u, v)


def test_batchnorm1d_input_matches_the_oracle():
    """A [N, C, L] input against the fp64 oracle: forward on the same x bits,
    backward on the module's own y bits."""
    wl = workloads.config(2).with_shape(8, 24, 50, 1)
    inp = workloads.make_inputs(wl)
    m = _module(wl, inp)
    x_leaf = harness.to_device(inp.x, wl).reshape(8, 24, 50).requires_grad_()
    y = m(x_leaf.clone())
    dy = harness.to_device(inp.dy, wl).reshape(8, 24, 50)
    y.backward(dy)
    torch.cuda.synchronize()
    a = harness.f32(wl.act_param)
    f = oracle.forward_train(harness.storage_channels(inp.x, wl), inp.gamma, inp.beta, wl.act, a,
                             harness.f32(wl.eps), harness.f32(wl.momentum), inp.running_mean,
                             inp.running_var, storage=wl.dtype)
    yg = harness.to_nchw64(y.detach().reshape(8, 24, 50, 1), wl)
    o = oracle.backward_from_y(yg, harness.storage_channels(inp.dy, wl), inp.gamma, inp.beta,
                               f["invstd"], wl.act, a)
    err = {"y": harness.rel_err_tensor(yg, f["y"]),
           "running_var": harness.rel_err_vec(m.running_var.cpu().numpy(), f["running_var"]),
           "dx": harness.rel_err_tensor(harness.to_nchw64(x_leaf.grad.reshape(8, 24, 50, 1), wl),
                                        o["dx"]),
           "dgamma": harness.rel_err_vec(m.weight.grad.cpu().numpy(), o["dgamma"]),
           "dbeta": harness.rel_err_vec(m.bias.grad.cpu().numpy(), o["dbeta"])}
    print("1d:", err, flush=True)
    harness.assert_within(err, wl.dtype, "1d")


def _torch_ref(N, C, H, W, **bn):
    """torch CPU fp64 BatchNorm2d + leaky ReLU with the same options (a library
    cross-check of the module's options, not of the kernels)."""
    return torch.nn.Sequential(torch.nn.BatchNorm2d(C, dtype=torch.float64, **bn),
                               torch.nn.LeakyReLU(0.01))


def _rel(a, b):
    a = a.detach().double().cpu()
    b = b.detach().double().cpu()
    return float((a - b).abs().max() / (b.abs().max() + 1e-30))


def test_module_options_follow_batchnorm2d():
    """momentum=None (cumulative average over the steps), affine=False, and
    track_running_stats=False (batch statistics in eval mode too) behave as in
    BatchNorm2d + LeakyReLU, within fp32 rounding of torch's fp64 result."""
    N, C, H, W = 4, 8, 10, 12
    g = torch.Generator().manual_seed(5)
    xs = [torch.randn(N, C, H, W, generator=g) * 2 + 1 for _ in range(3)]
    # cumulative average of the running statistics over three training steps
    m = InPlaceABN(C, momentum=None, device="cuda")
    ref = _torch_ref(N, C, H, W, momentum=None)
    for x in xs:
        m(x.cuda())
        ref(x.double())
    assert int(m.num_batches_tracked) == 3
    assert _rel(m.running_mean, ref[0].running_mean) < 1e-5
    assert _rel(m.running_var, ref[0].running_var) < 1e-5
    # without the affine step, weight and bias are fixed buffers
    m = InPlaceABN(C, affine=False, device="cuda")
    assert not any(True for _ in m.parameters())
    ref = _torch_ref(N, C, H, W, affine=False)
    x = xs[0].cuda().requires_grad_()
    y = m(x.clone())
    y.backward(torch.ones_like(y))
    xr = xs[0].double().requires_grad_()
    yr = ref(xr)
    yr.backward(torch.ones_like(yr))
    assert _rel(y, yr) < 1e-5 and _rel(x.grad, xr.grad) < 1e-4
    # no running statistics: eval mode normalises with the batch's own
    m = InPlaceABN(C, track_running_stats=False, device="cuda").eval()
    ref = _torch_ref(N, C, H, W, track_running_stats=False).eval()
    assert m.running_mean is None
    y = m(xs[1].cuda())
    assert _rel(y, ref(xs[1].double())) < 1e-5

"""iabn_forward_train_noalloc (the training forward with the library's static
scratch as workspace) against iabn_forward_train with a caller's workspace,
through the C ABI: bit-identical outputs on calls in a row on one device, each
smaller than the one before, and within the parity tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import harness
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import place_batchnorm_activation_amd as iabn

CODES = {"NCHW": 0, "NHWC": 1}
DT = {"f32": 0, "bf16": 1, "f16": 2}
ACT = {"identity": 0, "leaky_relu": 1, "elu": 2}

# largest first: grouped NHWC with its exchange in the scratch, then smaller ones
# (a channel group per NCHW channel, the split path, a resident one)
CASES = [workloads.config(3).with_shape(2, 256, 256, 256),
         workloads.config(5),
         workloads.config(2).with_shape(3, 64, 112, 112),
         workloads.config(3).with_shape(2, 64, 80, 80),
         workloads.config(1)]


def _call(noalloc: bool, inp, ws=None):
    wl = inp.wl
    x = harness.to_device(inp.x, wl)
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    rm = torch.from_numpy(inp.running_mean).cuda()
    rv = torch.from_numpy(inp.running_var).cuda()
    sm, si = torch.empty(wl.C, device="cuda"), torch.empty(wl.C, device="cuda")
    args = [x.data_ptr(), wl.N, wl.C, wl.H, wl.W, CODES[wl.layout], DT[wl.dtype], g.data_ptr(),
            b.data_ptr(), rm.data_ptr(), rv.data_ptr(), sm.data_ptr(), si.data_ptr(),
            ACT[wl.act], ctypes.c_float(wl.act_param), ctypes.c_float(wl.eps),
            ctypes.c_float(wl.momentum)]
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = iabn.lib.iabn_forward_train_noalloc(*args, stream)
    else:
        st = iabn.lib.iabn_forward_train(*args, ws.data_ptr(), ws.numel(), stream)
    assert st == 0, iabn.status_string(st)
    torch.cuda.synchronize()
    return {"y": x, "save_mean": sm, "save_invstd": si, "running_mean": rm, "running_var": rv}


def test_noalloc_forward_matches_workspace_forward():
    sizes = []
    for wl in CASES:
        sizes.append(wl.storage_bytes)
        inp = workloads.make_inputs(wl)
        plan = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                       workloads.storage_torch_dtype(wl.dtype), wl.act)
        need = iabn.iabn_workspace_size(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                        workloads.storage_torch_dtype(wl.dtype))
        print("case:", wl.name, wl.N, wl.C, wl.H, wl.W, plan, "workspace", need, flush=True)
        assert 0 < need <= iabn.NOALLOC_SCRATCH_BYTES
        ws = iabn.workspace(wl.N, wl.C, wl.H, wl.W, wl.layout,
                            workloads.storage_torch_dtype(wl.dtype))
        ref = _call(False, inp, ws)
        got = _call(True, inp)
        for k in ref:
            assert torch.equal(got[k], ref[k]), (wl.name, k)
        # and the oracle's bar on the same input
        run = harness.GpuRun(y=got["y"], dx=None,
                             save_mean=got["save_mean"].cpu().numpy(),
                             save_invstd=got["save_invstd"].cpu().numpy(),
                             running_mean=got["running_mean"].cpu().numpy(),
                             running_var=got["running_var"].cpu().numpy(),
                             dgamma=None, dbeta=None)
        errs = harness.check_forward(inp, run)
        print("  ", errs, flush=True)
        harness.assert_within(errs, wl.dtype, wl.name)
    assert all(a > b for a, b in zip(sizes, sizes[1:]))          # each call smaller


def test_noalloc_forward_twice_on_the_same_input():
    """Two calls in a row on one input (the scratch keeps the first call's words):
    the same bits."""
    wl = workloads.config(5)
    inp = workloads.make_inputs(wl)
    a = _call(True, inp)
    b = _call(True, inp)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _prepared(inp):
    wl = inp.wl
    d = {"x0": harness.to_device(inp.x, wl), "g": torch.from_numpy(inp.gamma).cuda(),
         "b": torch.from_numpy(inp.beta).cuda(),
         "rm0": torch.from_numpy(inp.running_mean).cuda(),
         "rv0": torch.from_numpy(inp.running_var).cuda()}
    d["x"], d["rm"], d["rv"] = d["x0"].clone(), d["rm0"].clone(), d["rv0"].clone()
    d["sm"], d["si"] = torch.empty(wl.C, device="cuda"), torch.empty(wl.C, device="cuda")
    return d


def _reset(d):
    d["x"].copy_(d["x0"])
    d["rm"].copy_(d["rm0"])
    d["rv"].copy_(d["rv0"])
    d["sm"].fill_(float("nan"))
    d["si"].fill_(float("nan"))


def _noalloc(wl, d, stream):
    st = iabn.lib.iabn_forward_train_noalloc(
        d["x"].data_ptr(), wl.N, wl.C, wl.H, wl.W, CODES[wl.layout], DT[wl.dtype],
        d["g"].data_ptr(), d["b"].data_ptr(), d["rm"].data_ptr(), d["rv"].data_ptr(),
        d["sm"].data_ptr(), d["si"].data_ptr(), ACT[wl.act], ctypes.c_float(wl.act_param),
        ctypes.c_float(wl.eps), ctypes.c_float(wl.momentum), stream)
    assert st == 0, iabn.status_string(st)


def test_noalloc_forward_graph_replays_match_eager():
    """The entry point is for callers that cannot allocate, such as code under
    graph capture: captured once, replayed four times, with an eager call of
    another shape (another plan over the same scratch) between the replays;
    every replay gives the eager call's bits."""
    wl = workloads.config(3).with_shape(2, 256, 128, 128)      # grouped NHWC
    other = workloads.config(2).with_shape(3, 64, 56, 56)      # NCHW, channel groups
    inp, inp_o = workloads.make_inputs(wl), workloads.make_inputs(other)
    d, e = _prepared(inp), _prepared(inp_o)
    print("case:", wl.name, iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                                    d["x"].dtype, wl.act), flush=True)
    _reset(d)
    _noalloc(wl, d, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    OUT = ("x", "rm", "rv", "sm", "si")
    eager = {k: d[k].clone() for k in OUT}
    _reset(e)
    _noalloc(other, e, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager_o = {k: e[k].clone() for k in OUT}
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    _reset(d)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        _noalloc(wl, d, side.cuda_stream)
    for _ in range(4):
        _reset(d)
        _reset(e)
        _noalloc(other, e, torch.cuda.current_stream().cuda_stream)   # eager, same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in OUT:
            assert torch.equal(d[k], eager[k]), k
            assert torch.equal(e[k], eager_o[k]), k

"""The library's calls inside a captured HIP graph (GPU).

The kernels allocate nothing and issue no memset, so a step can be captured once
and replayed; the slice-resident groups tag their exchange with an epoch kept in
the workspace, so every replay runs with a fresh token.  Each test captures a forward + backward on a side stream, then
replays it several times with eager work in between (restoring the in-place
input and the running statistics) and checks every replay bit for bit against
the eager run of the same calls.  One case per kernel family.
"""
import numpy as np
import pytest
import torch

import harness
import workloads

iabn = pytest.importorskip("place_batchnorm_activation_amd")

pytestmark = pytest.mark.gpu

CASES = [
    workloads.config(2).with_shape(4, 32, 16, 16),                 # NCHW channel-resident
    workloads.config(4).with_shape(4, 64, 28, 28),                 # ... ELU, z and dz kept
    workloads.config(2).with_shape(3, 64, 97, 100),                # ... channel groups of 2
    workloads.config(2).with_shape(3, 2, 300, 300),                # ... of 16, two levels
    workloads.config(5).with_shape(16, 512, 7, 7),                 # NHWC slice-resident, group 2
    workloads.config(3).with_shape(5, 256, 20, 20),                # ... group 4
    workloads.config(5),                                           # ... 8 lanes, group 8
    workloads.config(3).with_shape(5, 512, 50, 80),                # ... group 16, two levels
    workloads.config(3).with_shape(1, 256, 300, 300),              # streamed, group 64
    workloads.config(3).with_shape(2, 32, 96, 96),                 # NHWC split
    workloads.config(4).with_shape(2, 5, 17, 19),                  # NCHW resident, elements
    workloads.config(4).with_shape(2, 3, 150, 151),                # NCHW split, scalar
]


def _bufs(wl, inp):
    C = wl.C
    d = dict(x0=harness.to_device(inp.x, wl), dy=harness.to_device(inp.dy, wl),
             g=torch.from_numpy(inp.gamma).cuda(), b=torch.from_numpy(inp.beta).cuda(),
             rm0=torch.from_numpy(inp.running_mean).cuda(),
             rv0=torch.from_numpy(inp.running_var).cuda())
    d["x"] = d["x0"].clone()
    d["dx"] = torch.empty_like(d["dy"])
    d["rm"], d["rv"] = d["rm0"].clone(), d["rv0"].clone()
    for k in ("sm", "si", "dg", "db"):
        d[k] = torch.empty(C, device="cuda")
    d["ws"] = iabn.workspace(wl.N, C, wl.H, wl.W, wl.layout, d["x"].dtype)
    return d


def _train_step(wl, d, stream):
    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    iabn.iabn_forward_train(d["x"], N, C, H, W, wl.layout, d["g"], d["b"], d["rm"], d["rv"],
                            d["sm"], d["si"], wl.act, wl.act_param, wl.eps, wl.momentum, d["ws"],
                            stream)
    iabn.iabn_backward(d["x"], d["dy"], d["dx"], N, C, H, W, wl.layout, d["g"], d["b"], d["si"],
                       d["dg"], d["db"], wl.act, wl.act_param, d["ws"], stream)


def _reset(d):
    d["x"].copy_(d["x0"])
    d["rm"].copy_(d["rm0"])
    d["rv"].copy_(d["rv0"])
    d["dx"].fill_(float("nan"))
    for k in ("sm", "si", "dg", "db"):
        d[k].fill_(float("nan"))


OUTS = ("x", "dx", "sm", "si", "dg", "db", "rm", "rv")


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_train_step_graph_replays_match_eager(wl):
    inp = workloads.make_inputs(wl)
    d = _bufs(wl, inp)
    _reset(d)
    _train_step(wl, d, None)
    torch.cuda.synchronize()
    eager = {k: d[k].clone() for k in OUTS}
    print("case:", wl.name, iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                                    d["x"].dtype, wl.act), flush=True)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    _reset(d)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        _train_step(wl, d, side.cuda_stream)
    for _ in range(4):
        _reset(d)                                  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(d[k], eager[k]), k


def test_frozen_step_graph_replays_match_eager():
    wl = workloads.config(3).with_shape(2, 64, 40, 40)
    inp = workloads.make_inputs(wl)
    d = _bufs(wl, inp)
    rng = np.random.default_rng(8)
    d["rv0"].copy_(torch.from_numpy(rng.uniform(0.5, 2, wl.C).astype(np.float32)))
    N, C, H, W = wl.N, wl.C, wl.H, wl.W

    def step(stream):
        iabn.iabn_forward_eval(d["x"], N, C, H, W, wl.layout, d["g"], d["b"], d["rm"], d["rv"],
                               wl.act, wl.act_param, wl.eps, stream)
        iabn.iabn_backward_eval(d["x"], d["dy"], d["dx"], N, C, H, W, wl.layout, d["g"], d["b"],
                                d["rv"], wl.eps, d["dg"], d["db"], wl.act, wl.act_param, d["ws"],
                                stream)

    _reset(d)
    step(None)
    torch.cuda.synchronize()
    eager = {k: d[k].clone() for k in ("x", "dx", "dg", "db")}
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    _reset(d)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        step(side.cuda_stream)
    for _ in range(4):
        _reset(d)
        graph.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(d[k], eager[k]), k


CKPT_CASES = [
    workloads.config(2).with_shape(4, 32, 16, 16),                 # NCHW
    workloads.config(4).with_shape(2, 16, 40, 40),                 # NCHW f16, ELU
    workloads.config(3).with_shape(3, 64, 24, 24),                 # NHWC bf16
]


@pytest.mark.parametrize("wl", CKPT_CASES, ids=lambda w: w.name)
def test_ckpt_step_graph_replays_match_eager(wl):
    """Optimized checkpointing captured as one step: the forward keeping xhat,
    the recompute of y from xhat, the backward from xhat."""
    inp = workloads.make_inputs(wl)
    d = _bufs(wl, inp)
    d["y"], d["yr"] = torch.empty_like(d["x"]), torch.empty_like(d["x"])
    N, C, H, W = wl.N, wl.C, wl.H, wl.W

    def step(stream):
        iabn.iabn_forward_train_ckpt(d["x"], d["y"], N, C, H, W, wl.layout, d["g"], d["b"],
                                     d["rm"], d["rv"], d["sm"], d["si"], wl.act, wl.act_param,
                                     wl.eps, wl.momentum, d["ws"], stream)
        iabn.iabn_recompute_from_xhat(d["x"], d["yr"], N, C, H, W, wl.layout, d["g"], d["b"],
                                      wl.act, wl.act_param, stream)
        iabn.iabn_backward_ckpt(d["x"], d["dy"], d["dx"], N, C, H, W, wl.layout, d["g"],
                                d["b"], d["si"], d["dg"], d["db"], wl.act, wl.act_param,
                                d["ws"], stream)

    def reset():
        _reset(d)
        d["y"].fill_(float("nan"))
        d["yr"].fill_(float("nan"))

    outs = OUTS + ("y", "yr")
    reset()
    step(None)
    torch.cuda.synchronize()
    eager = {k: d[k].clone() for k in outs}
    assert torch.equal(eager["y"], eager["yr"])
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        step(side.cuda_stream)
    for _ in range(4):
        reset()
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(d[k], eager[k]), k

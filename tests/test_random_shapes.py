"""GPU parity on seeded random shapes: every layout, storage dtype and activation,
channel counts with and without 16-byte rows, maps from one row to a few
million elements.  Whatever kernels the plan picks for a shape (channel- or
slice-resident, grouped, streamed, split, scalar) must match the fp64 oracle
within the same gates as the fixed cases, and the plan reported must name the
kernels of one of those families.
"""
import dataclasses

import numpy as np
import pytest
import torch

import harness
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import place_batchnorm_activation_amd as iabn

FAMILIES = ("channel_resident", "channel_resident_scalar", "slice_resident", "slice_streamed",
            "split")
ACTS = (("leaky_relu", 0.01), ("leaky_relu", 0.2), ("elu", 1.0), ("elu", 0.5),
        ("identity", 0.0))


def _cases(n=48, seed=20241203, max_numel=3_000_000):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        layout = ("NCHW", "NHWC")[rng.integers(2)]
        dtype = ("f32", "bf16", "f16")[rng.integers(3)]
        act, p = ACTS[rng.integers(len(ACTS))]
        # channel counts: multiples of 8 (16-byte rows in every dtype) and others
        C = int(8 * rng.integers(1, 80)) if rng.random() < 0.7 else int(rng.integers(1, 300))
        N = int(rng.integers(1, 9))
        H = int(rng.integers(1, 80))
        W = int(rng.integers(1, 80))
        numel = N * C * H * W
        if N * H * W < 2 or numel > max_numel:
            continue
        base = 4 if act == "elu" else (2 if dtype == "f32" else 3)
        wl = workloads.config(base).with_shape(N, C, H, W)
        wl = dataclasses.replace(wl, layout=layout, dtype=dtype, act=act, act_param=p,
                                 name="rand%02d_%s_%s_%s_%dx%dx%dx%d" % (len(out), layout, dtype,
                                                                           act, N, C, H, W))
        out.append(wl)
    return out


def _big_nhwc_cases(n=10, seed=7, max_numel=40_000_000):
    """NHWC maps of 10 to 40 million elements with 16-byte rows: grouped
    slice-resident, streamed (register, LDS and re-read rows) and split plans."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = ("f32", "bf16", "f16")[rng.integers(3)]
        act, p = ACTS[rng.integers(len(ACTS))]
        C = int((64, 128, 256, 512, 1024, 2048)[rng.integers(6)])
        N = int(rng.integers(1, 5))
        H = int(rng.integers(20, 400))
        W = int(rng.integers(20, 400))
        numel = N * C * H * W
        if numel < 10_000_000 or numel > max_numel:
            continue
        base = 4 if act == "elu" else (2 if dtype == "f32" else 3)
        wl = workloads.config(base).with_shape(N, C, H, W)
        wl = dataclasses.replace(wl, layout="NHWC", dtype=dtype, act=act, act_param=p,
                                 name="big%02d_NHWC_%s_%s_%dx%dx%dx%d" % (len(out), dtype, act,
                                                                           N, C, H, W))
        out.append(wl)
    return out


CASES = _cases() + _big_nhwc_cases()


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_random_shape(wl):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    print("case:", wl.name, desc, flush=True)
    for part in desc.split():
        fam = part.split("=", 1)[1].split("(", 1)[0]
        assert fam in FAMILIES, desc
    inp = workloads.make_inputs(wl)
    run = harness.run_gpu(inp)
    ef = harness.check_forward(inp, run)
    eb = harness.check_backward(inp, run, dx_scale="terms" if wl.m == 2 else "rms")
    print("  forward", ef, "\n  backward", eb, flush=True)
    harness.assert_within(ef, wl.dtype, "forward " + wl.name)
    harness.assert_within(eb, wl.dtype, "backward " + wl.name)

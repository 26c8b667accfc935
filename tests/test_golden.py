"""Regression pin: the oracle and the input generator still reproduce the stored
snapshot written by tests/golden/make_golden.py (CPU only)."""
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "tiny_nchw_f32_leaky.json")


def test_oracle_reproduces_snapshot():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    wl = workloads.config(1)
    inp = workloads.make_inputs(wl)
    shape = tuple(g["shape_nchw"])
    x = workloads.from_storage(inp.x, *shape, wl.layout, wl.dtype)
    dy = workloads.from_storage(inp.dy, *shape, wl.layout, wl.dtype)
    assert np.array_equal(x.reshape(-1), np.array(g["x"]))
    assert np.array_equal(dy.reshape(-1), np.array(g["dy"]))
    f = oracle.forward_train(x, g["gamma"], g["beta"], g["act"], g["act_param"], g["eps"],
                             g["momentum"], inp.running_mean, inp.running_var, storage="f32")
    b = oracle.backward_from_y(f["y"], dy, g["gamma"], g["beta"], f["invstd"], g["act"],
                               g["act_param"])
    for key, val in (("y_f32", f["y"]), ("mean", f["mean"]), ("invstd", f["invstd"]),
                     ("running_mean", f["running_mean"]), ("running_var", f["running_var"]),
                     ("dx", b["dx"]), ("dgamma", b["dgamma"]), ("dbeta", b["dbeta"])):
        ref = np.array(g[key])
        assert np.allclose(val.reshape(-1), ref, rtol=1e-14, atol=1e-14 * np.abs(ref).max()), key

"""Write tests/golden/tiny_nchw_f32_leaky.json: the seeded 2x4x8x8 fp32 NCHW leaky-ReLU
workload and the fp64 oracle's outputs on it.  Calls only oracle/ (and the input
generator); no value here comes from the HIP library.  A regression snapshot: a later
change to the oracle's arithmetic must say why in its commit and regenerate this file.

The pages print no worked example, so nothing here is quoted from them; the method is
the training forward and the from-y backward of In-Place Activated BatchNorm (paperlayer
summary, section 3)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    wl = workloads.config(1)
    inp = workloads.make_inputs(wl)
    x = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    dy = workloads.from_storage(inp.dy, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    f = oracle.forward_train(x, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps, wl.momentum,
                             inp.running_mean, inp.running_var, storage="f32")
    b = oracle.backward_from_y(f["y"], dy, inp.gamma, inp.beta, f["invstd"], wl.act, wl.act_param)
    out = {
        "what": "oracle outputs on the seeded tiny workload (regression snapshot)",
        "shape_nchw": [wl.N, wl.C, wl.H, wl.W], "act": wl.act, "act_param": wl.act_param,
        "eps": wl.eps, "momentum": wl.momentum, "seed": 1000 + wl.index,
        "x": x.reshape(-1).tolist(), "dy": dy.reshape(-1).tolist(),
        "gamma": inp.gamma.astype(float).tolist(), "beta": inp.beta.astype(float).tolist(),
        "y_f32": f["y"].reshape(-1).tolist(), "mean": f["mean"].tolist(),
        "invstd": f["invstd"].tolist(), "running_mean": f["running_mean"].tolist(),
        "running_var": f["running_var"].tolist(),
        "dx": b["dx"].reshape(-1).tolist(), "dgamma": b["dgamma"].tolist(),
        "dbeta": b["dbeta"].tolist(),
    }
    path = os.path.join(HERE, "tiny_nchw_f32_leaky.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=0)
    print(path)


if __name__ == "__main__":
    main()

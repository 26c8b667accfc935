"""Benchmark of the In-Place ABN hot path on one MI355X.

One step = one training forward (statistics + normalise/activate in place) and
one backward (reductions from y + dx) over one batch of synthetic input already
resident in HBM, all through the C ABI.

  python bench.py [--steps K] [--warmup W] [--config I] [--gpus 1] [--no-cpu]
                  [--dtype f32|bf16|f16] [--mode train|frozen|block|shapes|ckpt]

The default workload is the largest single-GPU one, the 2x256x512x512 bf16 NHWC
segmentation-scale feature map (leaky ReLU 0.01).

Prints ONE JSON line.  value = numel / time-per-step (Gelem/s), measured "cold":
consecutive steps rotate over buffer sets totalling >= 512 MB, more than the
256 MB Infinity Cache, so every step reads its tensors from HBM.  The same loop
on one buffer set is reported as "warm".

Byte models (S = tensor bytes):
  minimal   forward 2S (read x, write y), backward 3S (read y and dy, write dx):
            5S per step.  The roofline's "achieved" figure and "min_bytes_GBps"
            use it: no kernel can move less.
  pass      forward 3S, backward 5S (each reduction pass re-reads its inputs):
            8S per step, reported as "pass_model_GBps" only; kernels that keep
            the tensor on chip between their passes move less than this, so the
            figure is not a bandwidth.
  counters  rocprofv3 FETCH_SIZE + WRITE_SIZE of the dominant kernel, calibrated
            on a plain copy ("roofline.traffic", "roofline.hbm_GBps").

The roofline object is for the dominant kernel (the longest average duration),
timed with HIP events recorded on the stream the library launches on (torch's
current stream) around each single-kernel call in further timed loops over the
same buffer sets.

--dtype stores the workload in another storage dtype.  --mode frozen measures
the step of a network fine-tuned with frozen normalisation statistics instead:
iabn_forward_eval (read x, write y: 2S) + iabn_backward_eval with dgamma/dbeta
(read y and dy, write dx in the same pass as the sums: 3S), 5S per step.

--mode block compares, on the workload's tensor, a chain of L layers of
(1x1 convolution -> normalisation + activation) built with the InPlace-ABN
autograd module against the same chain with torch's BatchNorm2d + activation:
forward + backward time per iteration, activation memory held after the
forward, and peak memory (the pages' claims: less training memory at a small
compute cost).  The convolutions are torch's (MIOpen) in both chains.

--mode ckpt times InPlace-ABN II against optimized checkpointing (the block keeps
xhat), the comparison the pages make.

--mode shapes checks the plan on ResNet-50 activation shapes (N = 32 and a few
others, NCHW fp32 and NHWC bf16): the cold step with the kernels the plan picks
against the split kernels (the stage entry points), one JSON line per shape.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD public figure
METRIC = "InPlace-ABN fwd+bwd Gelem/s and achieved HBM GB/s (% of MI355X peak)"
COLD_BYTES = 512 << 20


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed, so that
    an edit of comments alone leaves the digest as it was."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                 # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """Digest of the kernel sources' code (comments excluded): the counter figures
    in profiles/traffic.json hold for the kernels built from code with this digest."""
    h = hashlib.sha256()
    for f in ("device.hpp", "plan.hpp", "fused.hpp", "group.hpp", "fwd.hip", "bwd.hip",
              "fused_nchw.hip", "fused_nhwc.hip", "ckpt.hip", "noalloc.hip"):
        with open(os.path.join(ROOT, "place_batchnorm_activation_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        table = json.load(fh)
    ent = table.get("%s@%s" % (kernel, workload))
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (lscpu's "Model name", from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _rel_err(g: np.ndarray, o: np.ndarray, per_channel: bool) -> float:
    """max_i |g_i - o_i| / (|o_i| + rms(o)), the RMS over the element's channel
    (per_channel: [N, C, H, W] arrays) or over the whole vector."""
    if g.size == 0:
        return 0.0
    if per_channel:
        rms = np.sqrt(np.mean(o * o, axis=(0, 2, 3), keepdims=True))
    else:
        rms = np.sqrt(np.mean(o * o))
    return float(np.max(np.abs(g - o) / (np.abs(o) + rms + 1e-300)))


def cpu_baseline(wl, inp, gpu=None) -> dict:
    """The fp64 oracle, as it stands, on the host cores: forward + from-y backward,
    timed on a bounded sample of whole channels.  With `gpu` (the outputs of one
    step of the HIP path on the same input), also the largest error of each
    output on those channels against the oracle: the forward on the same x bits,
    the backward on the GPU's own y bits and save_invstd."""
    import oracle
    import workloads
    x = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    dy = workloads.from_storage(inp.dy, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    # bounded sample: whole channels, enough for ~10 s of oracle work
    per_elem_guess = 4e-8 / max(1, oracle.num_threads())
    ch = int(min(wl.C, max(1, 10.0 / (per_elem_guess * wl.m) / 3)))
    xs, dys = np.ascontiguousarray(x[:, :ch]), np.ascontiguousarray(dy[:, :ch])
    del x, dy
    g, b = inp.gamma[:ch], inp.beta[:ch]
    f32 = lambda v: float(np.float32(v))               # the scalars the library receives
    a, eps, mom = f32(wl.act_param), f32(wl.eps), f32(wl.momentum)
    # repeated until about 10 s of oracle work (at least 3 runs, at most 200)
    times = []
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 200):
        t0 = time.perf_counter()
        f = oracle.forward_train(xs, g, b, wl.act, a, eps, mom, inp.running_mean[:ch],
                                 inp.running_var[:ch], storage=wl.dtype)
        oracle.backward_from_y(f["y"], dys, g, b, f["invstd"], wl.act, a)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    n = ch * wl.m
    out = {"value": round(n / t / 1e9, 5), "unit": "Gelem/s", "cores": oracle.num_threads(),
           "cpu_model": cpu_model(), "kind": "oracle",
           "sample": "%d of %d channels (all %d elements each) of the same workload, fp64 "
                     "forward_train + backward_from_y, median of %d runs (%.3f s each, "
                     "%.1f s in all)" % (ch, wl.C, wl.m, len(times), t, sum(times))}
    if gpu is not None:
        y = gpu["y"][:, :ch]
        err = {"y": _rel_err(y, f["y"], True)}
        for k, ok in (("save_mean", "mean"), ("save_invstd", "invstd"),
                      ("running_mean", "running_mean"), ("running_var", "running_var")):
            err[k] = _rel_err(gpu[k][:ch].astype(np.float64), f[ok], False)
        o = oracle.backward_from_y(np.ascontiguousarray(y), dys, g, b,
                                   gpu["save_invstd"][:ch].astype(np.float64), wl.act, a)
        err["dx"] = _rel_err(gpu["dx"][:, :ch], o["dx"], True)
        err["dgamma"] = _rel_err(gpu["dgamma"][:ch].astype(np.float64), o["dgamma"], False)
        err["dbeta"] = _rel_err(gpu["dbeta"][:ch].astype(np.float64), o["dbeta"], False)
        out["max_rel_err"] = {k: float("%.3g" % v) for k, v in err.items()}
        out["max_rel_err_channels"] = ch
    return out


def run_frozen(args, wl) -> int:
    """Steps of iabn_forward_eval + iabn_backward_eval (frozen running statistics)."""
    import torch
    import place_batchnorm_activation_amd as iabn
    import workloads

    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    inp = workloads.make_inputs(wl)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sshape = (N, C, H, W) if wl.layout == "NCHW" else (N, H, W, C)
    S = wl.storage_bytes
    nsets = max(2, math.ceil(COLD_BYTES / (3 * S)))
    x0 = workloads.to_torch(inp.x, wl.dtype).reshape(sshape).to(dev)
    dy0 = workloads.to_torch(inp.dy, wl.dtype).reshape(sshape).to(dev)
    sets = [{"x": x0.clone(), "dy": dy0.clone(), "dx": torch.empty_like(dy0)}
            for _ in range(nsets)]
    g = torch.from_numpy(inp.gamma).to(dev)
    b = torch.from_numpy(inp.beta).to(dev)
    # frozen statistics with running_var = gamma^2 - eps and running_mean = beta: the
    # in-place forward then maps x to +-(x - beta) + beta, so repeated steps on a
    # buffer set keep its values bounded
    rm = b.clone()
    rv = torch.from_numpy(np.maximum(inp.gamma.astype(np.float64) ** 2 - wl.eps, 1e-2)
                          .astype(np.float32)).to(dev)
    dg, db = torch.empty(C, device=dev), torch.empty(C, device=dev)
    ws = iabn.workspace(N, C, H, W, wl.layout, x0.dtype, dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def fwd(s):
        iabn.iabn_forward_eval(s["x"], N, C, H, W, wl.layout, g, b, rm, rv, wl.act, wl.act_param,
                               wl.eps, sp)

    def bwd(s, grads=True):
        iabn.iabn_backward_eval(s["x"], s["dy"], s["dx"], N, C, H, W, wl.layout, g, b, rv, wl.eps,
                                dg if grads else None, db if grads else None, wl.act,
                                wl.act_param, ws, sp)

    def timed(calls, k):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(k):
            for fn in calls:
                fn(sets[i % nsets])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k          # us per step

    for i in range(args.warmup):
        fwd(sets[i % nsets])
        bwd(sets[i % nsets])
    us_step = timed([fwd, bwd], args.steps)
    us_fwd = timed([fwd], args.steps)
    us_bwd = timed([bwd], args.steps)
    us_dx = timed([lambda s: bwd(s, grads=False)], args.steps)
    # forward_eval is one kernel; backward_eval with the sums is one pass over y and
    # dy that writes dx, plus a small finishing kernel for dgamma/dbeta
    kernels = {"forward_eval": (us_fwd, 2 * S), "backward_eval": (us_bwd, 3 * S)}
    dom = max(kernels, key=lambda k: kernels[k][0])
    t_dom, dom_bytes = kernels[dom]
    achieved = dom_bytes / (t_dom * 1e-6) / 1e9
    gbps = 5 * S / (us_step * 1e-6) / 1e9
    out = {
        "metric": "InPlace-ABN frozen-statistics fwd+bwd Gelem/s",
        "value": round(wl.numel / (us_step * 1e-6) / 1e9, 4),
        "unit": "Gelem/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_step * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "C": C, "H": H, "W": W, "layout": wl.layout,
                   "storage": wl.dtype, "act": wl.act, "act_param": wl.act_param,
                   "mode": "frozen", "parallelism": "single_gpu"},
        "pass_model_GBps": round(gbps, 1),
        "pass_model_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "protocol": "cold: %d rotating buffer sets of %.0f MB; 5S per step" % (nsets, 3 * S / 1e6),
        "launch_us": {"forward_eval": round(us_fwd, 3), "backward_eval": round(us_bwd, 3),
                      "backward_eval_dx_only": round(us_dx, 3), "step": round(us_step, 3)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(t_dom, 3)},
    }
    print(json.dumps(out), flush=True)
    return 0


SHAPES = [(32, 64, 112, 112), (32, 256, 56, 56), (32, 128, 56, 56), (32, 512, 28, 28),
          (32, 256, 28, 28), (32, 1024, 14, 14), (32, 256, 14, 14), (32, 2048, 7, 7),
          (32, 512, 7, 7), (8, 512, 28, 28), (8, 1024, 14, 14), (8, 2048, 7, 7),
          (64, 256, 14, 14)]


def run_shapes(args) -> int:
    """The plan's kernels (forward_train + backward) against the split kernels (the
    stage entry points) on ResNet-50 activation shapes, cold, one JSON line each."""
    import torch
    import place_batchnorm_activation_amd as iabn
    import workloads

    act, p, eps, mom = "leaky_relu", 0.01, 1e-5, 0.1
    for layout, dtype in (("NCHW", "f32"), ("NHWC", "bf16")):
        for (N, C, H, W) in SHAPES:
            wl = dataclasses.replace(workloads.config(2), N=N, C=C, H=H, W=W, layout=layout,
                                     dtype=dtype, name="resnet50_%dx%dx%dx%d" % (N, C, H, W))
            inp = workloads.make_device_inputs(wl, seed=5)
            S = wl.storage_bytes
            nsets = max(2, math.ceil(COLD_BYTES / (3 * S)))
            sets = [{"x": inp.x.clone(), "dy": inp.dy.clone(), "dx": torch.empty_like(inp.dy)}
                    for _ in range(nsets)]
            del inp.x, inp.dy
            g = torch.from_numpy(inp.gamma).cuda()
            b = torch.from_numpy(inp.beta).cuda()
            rm, rv = torch.zeros(C, device="cuda"), torch.ones(C, device="cuda")
            sm, si = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
            dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
            ws = iabn.workspace(N, C, H, W, layout, sets[0]["x"].dtype)

            def plan_step(s):
                iabn.iabn_forward_train(s["x"], N, C, H, W, layout, g, b, rm, rv, sm, si, act, p,
                                        eps, mom, ws)
                iabn.iabn_backward(s["x"], s["dy"], s["dx"], N, C, H, W, layout, g, b, si, dg,
                                   db, act, p, ws)

            def split_step(s):
                iabn.iabn_forward_stats(s["x"], N, C, H, W, layout, g, b, rm, rv, sm, si, eps,
                                        mom, ws)
                iabn.iabn_forward_apply(s["x"], N, C, H, W, layout, act, p, ws)
                iabn.iabn_backward_reduce(s["x"], s["dy"], N, C, H, W, layout, g, b, si, dg, db,
                                          act, p, ws)
                iabn.iabn_backward_apply(s["x"], s["dy"], s["dx"], N, C, H, W, layout, act, p,
                                         ws)

            def timed(fn, k=max(20, args.steps // 4)):
                for i in range(5):
                    fn(sets[i % nsets])
                torch.cuda.synchronize()
                # a short device-side wait lets the host queue the loop ahead, so that
                # small shapes are timed on the GPU rather than at Python's launch rate
                if hasattr(torch.cuda, "_sleep"):
                    torch.cuda._sleep(50_000_000)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(k):
                    fn(sets[i % nsets])
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / k

            t_plan, t_split = timed(plan_step), timed(split_step)
            plan = iabn.iabn_describe_plan(N, C, H, W, layout, sets[0]["x"].dtype, act)
            print(json.dumps({"mode": "shapes", "layout": layout, "storage": dtype,
                              "shape": [N, C, H, W], "plan": plan,
                              "plan_us": round(t_plan, 2), "split_us": round(t_split, 2),
                              "plan_pass_model_TBps": round(8 * S / t_plan / 1e6, 3)}),
                  flush=True)
            del sets
            torch.cuda.empty_cache()
    return 0


def run_ckpt(args, wl) -> int:
    """InPlace-ABN II against optimized checkpointing on the workload (the pages'
    comparison, paperlayer section 3): cold steps of
      ii_plan   iabn_forward_train + iabn_backward (the kernels the plan picks);
      ii_split  the same through the stage entry points (the split kernels);
      ckpt      iabn_forward_train_ckpt (xhat kept over x, y written) +
                iabn_recompute_from_xhat (y rebuilt for the next layer's backward) +
                iabn_backward_ckpt, on the split kernels as well.
    Minimal bytes: II 5S a step; checkpointing 8S (forward 3S: read x, write xhat
    and y; recompute 2S; backward 3S).  The split kernels move 8S (II) and 11S
    (checkpointing)."""
    import torch
    import place_batchnorm_activation_amd as iabn
    import workloads

    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    inp = workloads.make_inputs(wl)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sshape = (N, C, H, W) if wl.layout == "NCHW" else (N, H, W, C)
    S = wl.storage_bytes
    nsets = max(2, math.ceil(COLD_BYTES / (4 * S)))
    x0 = workloads.to_torch(inp.x, wl.dtype).reshape(sshape).to(dev)
    dy0 = workloads.to_torch(inp.dy, wl.dtype).reshape(sshape).to(dev)
    sets = [{"x": x0.clone(), "dy": dy0.clone(), "dx": torch.empty_like(dy0),
             "y": torch.empty_like(x0)} for _ in range(nsets)]
    g = torch.from_numpy(inp.gamma).to(dev)
    b = torch.from_numpy(inp.beta).to(dev)
    rm = torch.from_numpy(inp.running_mean).to(dev)
    rv = torch.from_numpy(inp.running_var).to(dev)
    sm, si = torch.empty(C, device=dev), torch.empty(C, device=dev)
    dg, db = torch.empty(C, device=dev), torch.empty(C, device=dev)
    ws = iabn.workspace(N, C, H, W, wl.layout, x0.dtype, dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    L, act, p, eps, mom = wl.layout, wl.act, wl.act_param, wl.eps, wl.momentum

    def ii_plan(s):
        iabn.iabn_forward_train(s["x"], N, C, H, W, L, g, b, rm, rv, sm, si, act, p, eps, mom,
                                ws, sp)
        iabn.iabn_backward(s["x"], s["dy"], s["dx"], N, C, H, W, L, g, b, si, dg, db, act, p,
                           ws, sp)

    def ii_split(s):
        iabn.iabn_forward_stats(s["x"], N, C, H, W, L, g, b, rm, rv, sm, si, eps, mom, ws, sp)
        iabn.iabn_forward_apply(s["x"], N, C, H, W, L, act, p, ws, sp)
        iabn.iabn_backward_reduce(s["x"], s["dy"], N, C, H, W, L, g, b, si, dg, db, act, p, ws,
                                  sp)
        iabn.iabn_backward_apply(s["x"], s["dy"], s["dx"], N, C, H, W, L, act, p, ws, sp)

    def ckpt(s):
        iabn.iabn_forward_train_ckpt(s["x"], s["y"], N, C, H, W, L, g, b, rm, rv, sm, si, act,
                                     p, eps, mom, ws, sp)
        iabn.iabn_recompute_from_xhat(s["x"], s["y"], N, C, H, W, L, g, b, act, p, sp)
        iabn.iabn_backward_ckpt(s["x"], s["dy"], s["dx"], N, C, H, W, L, g, b, si, dg, db, act,
                                p, ws, sp)

    def timed(fn, k):
        for i in range(max(3, args.warmup)):
            fn(sets[i % nsets])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(k):
            fn(sets[i % nsets])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k          # us per step

    res = {}
    for name, fn in (("ii_plan", ii_plan), ("ii_split", ii_split), ("ckpt", ckpt)):
        # each scheme twice, interleaved, and the better time kept
        res[name] = timed(fn, args.steps)
    for name, fn in (("ii_plan", ii_plan), ("ii_split", ii_split), ("ckpt", ckpt)):
        res[name] = min(res[name], timed(fn, args.steps))
    out = {
        "metric": "InPlace-ABN II vs optimized checkpointing, fwd+bwd us per step",
        "config": {"workload": wl.name, "N": N, "C": C, "H": H, "W": W, "layout": wl.layout,
                   "storage": wl.dtype, "act": wl.act, "act_param": wl.act_param,
                   "mode": "ckpt"},
        "data": "synthetic", "n_gpus": 1, "steps": args.steps,
        "protocol": "cold: %d rotating buffer sets of %.0f MB; best of two interleaved runs"
                    % (nsets, 4 * S / 1e6),
        "us_per_step": {k: round(v, 2) for k, v in res.items()},
        "gelem_per_s": {k: round(wl.numel / (v * 1e-6) / 1e9, 2) for k, v in res.items()},
        "ckpt_over_ii_split": round(res["ckpt"] / res["ii_split"], 4),
        "ckpt_over_ii_plan": round(res["ckpt"] / res["ii_plan"], 4),
        "plan": iabn.iabn_describe_plan(N, C, H, W, L, x0.dtype, act),
    }
    print(json.dumps(out), flush=True)
    return 0


def run_block(args, wl) -> int:
    """InPlace-ABN against BatchNorm2d + activation inside a convolution chain."""
    import torch
    import workloads
    from place_batchnorm_activation_amd.autograd import InPlaceABN

    N, C, H, W, L = wl.N, wl.C, wl.H, wl.W, args.layers
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    dt = workloads.storage_torch_dtype(wl.dtype)
    fmt = torch.channels_last if wl.layout == "NHWC" else torch.contiguous_format
    torch.manual_seed(0)
    convs = [torch.nn.Conv2d(C, C, 1, bias=False).to(dev, dt).to(memory_format=fmt)
             for _ in range(L)]
    act = {"leaky_relu": lambda: torch.nn.LeakyReLU(wl.act_param),
           "elu": lambda: torch.nn.ELU(wl.act_param), "identity": torch.nn.Identity}[wl.act]

    def torch_norm():
        bn = torch.nn.BatchNorm2d(C, eps=wl.eps, momentum=wl.momentum).to(dev)
        return torch.nn.Sequential(bn, act())

    chains = {
        "inplace_abn": [InPlaceABN(C, wl.eps, wl.momentum, wl.act, wl.act_param, device=dev)
                        for _ in range(L)],
        "batchnorm2d_act": [torch_norm() for _ in range(L)],
    }
    x = torch.randn(N, C, H, W, device=dev, dtype=dt).to(memory_format=fmt).requires_grad_()

    def step(norms):
        h = x
        for conv, norm in zip(convs, norms):
            h = norm(conv(h))
        h.backward(torch.ones_like(h))

    res = {}
    S = wl.storage_bytes
    for name, norms in chains.items():
        for _ in range(max(2, args.warmup // 5)):
            step(norms)
        torch.cuda.synchronize()
        # memory: activations held after the forward, and the peak of one iteration
        x.grad = None
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        h = x
        for conv, norm in zip(convs, norms):
            h = norm(conv(h))
        held = torch.cuda.memory_allocated() - base
        h.backward(torch.ones_like(h))
        del h
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        k = max(5, args.steps // 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(k):
            step(norms)
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"ms_per_iter": round(e0.elapsed_time(e1) / k, 4),
                     "held_after_forward_MB": round(held / 2**20, 1),
                     "held_tensors_per_layer": round(held / S / L, 2),
                     "peak_MB": round(peak / 2**20, 1), "iters": k}
        print("bench: block %s %s" % (name, res[name]), file=sys.stderr, flush=True)
    a, b = res["inplace_abn"], res["batchnorm2d_act"]
    out = {
        "metric": "conv1x1 + norm/act chain: InPlace-ABN vs BatchNorm2d+activation",
        "config": {"workload": wl.name, "N": N, "C": C, "H": H, "W": W, "layout": wl.layout,
                   "storage": wl.dtype, "act": wl.act, "act_param": wl.act_param, "layers": L,
                   "mode": "block"},
        "data": "synthetic", "n_gpus": 1,
        "inplace_abn": a, "batchnorm2d_act": b,
        "time_ratio": round(a["ms_per_iter"] / b["ms_per_iter"], 4),
        "held_memory_ratio": round(a["held_after_forward_MB"] / b["held_after_forward_MB"], 4),
        "peak_memory_ratio": round(a["peak_MB"] / b["peak_MB"], 4),
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index 1..5 (default 3, the largest)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--warm-only", action="store_true", help="one buffer set (for profiling)")
    ap.add_argument("--dtype", choices=("f32", "bf16", "f16"), default=None,
                    help="storage dtype instead of the workload's own")
    ap.add_argument("--mode", choices=("train", "frozen", "block", "shapes", "ckpt"),
                    default="train",
                    help="train: forward_train + backward; frozen: forward_eval + backward_eval; "
                         "block: conv + norm/act chain against torch's BatchNorm2d; "
                         "shapes: the plan's kernels against the split ones on ResNet-50 shapes; "
                         "ckpt: InPlace-ABN II against optimized checkpointing")
    ap.add_argument("--layers", type=int, default=4, help="layers of the --mode block chain")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark: copy a MIB-MiB buffer 5 times (a plain copy "
                         "kernel of known size, the reference that scales memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))
        return 0

    import place_batchnorm_activation_amd as iabn
    import workloads

    wl = workloads.config(args.config)
    if args.dtype and args.dtype != wl.dtype:
        wl = dataclasses.replace(wl, dtype=args.dtype, name="%s_as_%s" % (wl.name, args.dtype))
    if args.mode == "frozen":
        return run_frozen(args, wl)
    if args.mode == "block":
        return run_block(args, wl)
    if args.mode == "shapes":
        return run_shapes(args)
    if args.mode == "ckpt":
        return run_ckpt(args, wl)
    return run_train(args, wl)


# Minimal bytes of one launch of each single-kernel call, in units of S: a
# forward reads x and writes y, a backward reads y and dy and writes dx; the
# split path's elementwise kernels do the same.  The pass model charges a
# forward 3S and a backward 5S (its reductions re-read their inputs).
MIN_S = {"fwd": 2, "bwd": 3, "fwd_apply": 2, "bwd_apply": 3}
PASS_S = {"fwd": 3, "bwd": 5, "fwd_apply": 2, "bwd_apply": 3}


def run_train(args, wl) -> int:
    """Steps of iabn_forward_train + iabn_backward (the training hot path)."""
    import torch
    import place_batchnorm_activation_amd as iabn
    import workloads

    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    inp = workloads.make_inputs(wl)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sshape = (N, C, H, W) if wl.layout == "NCHW" else (N, H, W, C)
    S = wl.storage_bytes
    nsets = 1 if args.warm_only else max(2, math.ceil(COLD_BYTES / (3 * S)))

    x0 = workloads.to_torch(inp.x, wl.dtype).reshape(sshape).to(dev)
    dy0 = workloads.to_torch(inp.dy, wl.dtype).reshape(sshape).to(dev)
    sets = []
    for _ in range(nsets):
        sets.append({"x": x0.clone(), "dy": dy0.clone(), "dx": torch.empty_like(dy0)})
    warm_set = sets[0]
    g = torch.from_numpy(inp.gamma).to(dev)
    b = torch.from_numpy(inp.beta).to(dev)
    rm = torch.from_numpy(inp.running_mean).to(dev)
    rv = torch.from_numpy(inp.running_var).to(dev)
    sm, si = torch.empty(C, device=dev), torch.empty(C, device=dev)
    dg, db = torch.empty(C, device=dev), torch.empty(C, device=dev)
    ws = iabn.workspace(N, C, H, W, wl.layout, x0.dtype, dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def fwd(s):
        iabn.iabn_forward_train(s["x"], N, C, H, W, wl.layout, g, b, rm, rv, sm, si, wl.act,
                                wl.act_param, wl.eps, wl.momentum, ws, sp)

    def bwd(s):
        iabn.iabn_backward(s["x"], s["dy"], s["dx"], N, C, H, W, wl.layout, g, b, si, dg, db,
                           wl.act, wl.act_param, ws, sp)

    def step(s):
        fwd(s)
        bwd(s)

    def timed(set_list, k):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(k):
            step(set_list[i % len(set_list)])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k        # ms per step

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    print("bench: %s warmup done, %d buffer set(s)" % (wl.name, nsets), file=sys.stderr, flush=True)

    ms_cold = timed(sets, args.steps)
    ms_warm = timed([warm_set], args.steps)

    # Per-launch durations: HIP events recorded on the library's stream (torch's
    # current stream) around each call.  A fused pass is one kernel; with the split
    # path the single-kernel stages (the elementwise kernels) are timed through the
    # stage entry points.
    plan = iabn.iabn_describe_plan(N, C, H, W, wl.layout, x0.dtype, wl.act)
    fam_fwd = plan.split()[0].split("=", 1)[1].split("(", 1)[0]
    fam_bwd = plan.split()[1].split("=", 1)[1].split("(", 1)[0]
    fused_fwd = fam_fwd != "split"
    fused_bwd = fam_bwd != "split"

    def event_loop(calls):
        acc = np.zeros(len(calls))
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
               for _ in range(args.steps)]
        for i in range(args.steps):
            st = sets[i % nsets]
            evs[i][0].record(stream)
            for j, fn in enumerate(calls):
                fn(st)
                evs[i][j + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            for j in range(len(calls)):
                acc[j] += evs[i][j].elapsed_time(evs[i][j + 1])
        return [float(1e3 * a / args.steps) for a in acc]

    call_us = event_loop([fwd, bwd])
    timings = {"forward_train": round(call_us[0], 3), "backward": round(call_us[1], 3)}
    kernels = {}             # name -> (avg us, kind in MIN_S)
    if fused_fwd:
        kernels["fwd_" + fam_fwd] = (call_us[0], "fwd")
    if fused_bwd:
        kernels["bwd_" + fam_bwd] = (call_us[1], "bwd")
    if not (fused_fwd and fused_bwd):
        st_us = event_loop([
            lambda s: iabn.iabn_forward_stats(s["x"], N, C, H, W, wl.layout, g, b, rm, rv, sm,
                                              si, wl.eps, wl.momentum, ws, sp),
            lambda s: iabn.iabn_forward_apply(s["x"], N, C, H, W, wl.layout, wl.act,
                                              wl.act_param, ws, sp),
            lambda s: iabn.iabn_backward_reduce(s["x"], s["dy"], N, C, H, W, wl.layout, g, b, si,
                                                dg, db, wl.act, wl.act_param, ws, sp),
            lambda s: iabn.iabn_backward_apply(s["x"], s["dy"], s["dx"], N, C, H, W, wl.layout,
                                               wl.act, wl.act_param, ws, sp)])
        names = ["forward_stats", "forward_apply", "backward_reduce", "backward_apply"]
        timings.update({n: round(u, 3) for n, u in zip(names, st_us)})
        if not fused_fwd:
            kernels["fwd_apply"] = (st_us[1], "fwd_apply")
        if not fused_bwd:
            kernels["bwd_apply"] = (st_us[3], "bwd_apply")
    print("bench: %s; per-call us %s" % (plan, timings), file=sys.stderr, flush=True)
    dom = max(kernels, key=lambda k: kernels[k][0])
    t_dom_us, kind = kernels[dom]
    dom_bytes = MIN_S[kind] * S
    achieved = dom_bytes / (t_dom_us * 1e-6) / 1e9
    traffic = load_traffic(dom, wl.name)

    # One step on the original input, twice from the same state: the outputs the
    # oracle is compared with, and run-to-run bitwise determinism.
    def reference_step():
        s = {"x": x0.clone(), "dy": dy0.clone(), "dx": torch.empty_like(dy0)}
        rm1 = torch.from_numpy(inp.running_mean).to(dev)
        rv1 = torch.from_numpy(inp.running_var).to(dev)
        sm1, si1 = torch.empty(C, device=dev), torch.empty(C, device=dev)
        dg1, db1 = torch.empty(C, device=dev), torch.empty(C, device=dev)
        iabn.iabn_forward_train(s["x"], N, C, H, W, wl.layout, g, b, rm1, rv1, sm1, si1, wl.act,
                                wl.act_param, wl.eps, wl.momentum, ws, sp)
        iabn.iabn_backward(s["x"], s["dy"], s["dx"], N, C, H, W, wl.layout, g, b, si1, dg1, db1,
                           wl.act, wl.act_param, ws, sp)
        torch.cuda.synchronize()
        return {"y": s["x"], "dx": s["dx"], "save_mean": sm1, "save_invstd": si1,
                "running_mean": rm1, "running_var": rv1, "dgamma": dg1, "dbeta": db1}

    del sets
    r0, r1 = reference_step(), reference_step()
    deterministic = all(torch.equal(r0[k], r1[k]) for k in r0)
    del r1

    numel = wl.numel
    t = ms_cold * 1e-3
    out = {
        "metric": METRIC,
        "value": round(numel / t / 1e9, 4),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_cold, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "C": C, "H": H, "W": W, "layout": wl.layout,
                   "storage": wl.dtype, "act": wl.act, "act_param": wl.act_param,
                   "parallelism": "single_gpu"},
        "min_bytes_GBps": round(5 * S / t / 1e9, 1),
        "min_bytes_frac_of_peak": round(5 * S / t / 1e9 / HBM_PEAK_GBPS, 4),
        "pass_model_GBps": round(8 * S / t / 1e9, 1),
        "protocol": "cold: %d rotating buffer sets of %.0f MB" % (nsets, 3 * S / 1e6),
        "warm": {"ms_per_step": round(ms_warm, 5),
                 "value": round(numel / (ms_warm * 1e-3) / 1e9, 4),
                 "min_bytes_GBps": round(5 * S / (ms_warm * 1e-3) / 1e9, 1)},
        "deterministic": bool(deterministic),
        "plan": plan,
        "launch_us": timings,
        "roofline": {"kernel": dom, "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "hbm_GBps": (round(traffic / (t_dom_us * 1e-6) / 1e9, 1)
                                  if traffic else None),
                     "hbm_frac": (round(traffic / (t_dom_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                                  if traffic else None),
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "pass_model_bytes_per_launch": PASS_S[kind] * S,
                     "avg_launch_us": round(t_dom_us, 3)},
    }
    if not args.no_cpu:
        host = {}
        for k, v in r0.items():
            if v.dim() == 1:
                host[k] = v.cpu().numpy()
            else:
                host[k] = workloads.from_storage(workloads.from_torch(v, wl.dtype), N, C, H, W,
                                                 wl.layout, wl.dtype)
        del r0
        out["cpu_baseline"] = cpu_baseline(wl, inp, host)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Shared helpers of the parity tests and the smoke check: run the HIP path through
the binding, run the fp64 oracle on the same input bits, and compare.

Error metric (per tensor): max_i |g_i - o_i| / (|o_i| + rms_c(o)), where rms_c is
the RMS of the oracle's values over the channel of element i (for per-channel
vectors: over all C entries).  Gates: 1e-5 for fp32 storage, 2e-2 for bf16
storage (fp32 arithmetic in both cases), and for fp16 storage the bf16 gate
scaled by the ratio of the two formats' unit roundoffs (2^-11 / 2^-8): 2.5e-3.

Stage-wise gating: the forward is checked against the oracle run on the same x
bits; the backward against the oracle run on the GPU's own stored y bits and
save_invstd (the from-y backward is a function of exactly those).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import oracle
import workloads

TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2.5e-3}


def f32(v: float) -> float:
    """The fp32 value the library receives for a scalar argument."""
    return float(np.float32(v))


def rel_err_tensor(g: np.ndarray, o: np.ndarray) -> float:
    """g, o: fp64 [N, C, H, W]."""
    rms = np.sqrt(np.mean(o * o, axis=(0, 2, 3), keepdims=True))
    return float(np.max(np.abs(g - o) / (np.abs(o) + rms + 1e-300))) if g.size else 0.0


def rel_err_vec(g: np.ndarray, o: np.ndarray) -> float:
    rms = np.sqrt(np.mean(o * o))
    return float(np.max(np.abs(g - o) / (np.abs(o) + rms + 1e-300))) if g.size else 0.0


def storage_shape(wl: workloads.Workload) -> tuple:
    return (wl.N, wl.C, wl.H, wl.W) if wl.layout == "NCHW" else (wl.N, wl.H, wl.W, wl.C)


def to_device(a: np.ndarray, wl: workloads.Workload, device="cuda") -> torch.Tensor:
    return workloads.to_torch(a, wl.dtype).reshape(storage_shape(wl)).to(device)


def to_nchw64(t: torch.Tensor, wl: workloads.Workload, sel=None) -> np.ndarray:
    """A storage tensor (any device) -> fp64 logical-NCHW host array; with `sel` (a
    slice or index list of channels) only those channels are moved and widened."""
    if sel is None:
        return workloads.from_storage(workloads.from_torch(t, wl.dtype), wl.N, wl.C, wl.H, wl.W,
                                      wl.layout, wl.dtype)
    idx = _channel_index(sel, wl.C)
    if wl.layout == "NCHW":
        part = t[:, idx]
    else:
        part = t[..., idx]
    return workloads.from_storage(workloads.from_torch(part, wl.dtype), wl.N, len(idx), wl.H,
                                  wl.W, wl.layout, wl.dtype)


def storage_channels(a: np.ndarray, wl: workloads.Workload, sel=None) -> np.ndarray:
    """A host storage array (wl.layout) -> fp64 logical-NCHW array of the channels in
    `sel` (all when None), widened exactly."""
    if sel is None:
        return workloads.from_storage(a, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    idx = _channel_index(sel, wl.C)
    a = a.reshape(storage_shape(wl))
    part = a[:, idx] if wl.layout == "NCHW" else a[..., idx]
    return workloads.from_storage(np.ascontiguousarray(part), wl.N, len(idx), wl.H, wl.W,
                                  wl.layout, wl.dtype)


def _channel_index(sel, C: int):
    if isinstance(sel, slice):
        return list(range(C))[sel]
    return [int(c) for c in np.asarray(sel).reshape(-1)]


@dataclasses.dataclass
class GpuRun:
    y: torch.Tensor
    dx: Optional[torch.Tensor]
    save_mean: np.ndarray
    save_invstd: np.ndarray
    running_mean: np.ndarray
    running_var: np.ndarray
    dgamma: Optional[np.ndarray]
    dbeta: Optional[np.ndarray]


def run_gpu(inp: workloads.Inputs, backward: bool = True, dx_over_dy: bool = False,
            device="cuda", ws=None) -> GpuRun:
    """Training forward (in place) and backward through the C ABI (ws: a workspace
    to use instead of a fresh one)."""
    import place_batchnorm_activation_amd as iabn
    wl = inp.wl
    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    x = to_device(inp.x, wl, device)
    g = torch.from_numpy(inp.gamma).to(device)
    b = torch.from_numpy(inp.beta).to(device)
    rm = torch.from_numpy(inp.running_mean).to(device)
    rv = torch.from_numpy(inp.running_var).to(device)
    sm = torch.empty(C, device=device)
    si = torch.empty(C, device=device)
    if ws is None:
        ws = iabn.workspace(N, C, H, W, wl.layout, x.dtype, device)
    iabn.iabn_forward_train(x, N, C, H, W, wl.layout, g, b, rm, rv, sm, si, wl.act,
                            wl.act_param, wl.eps, wl.momentum, ws)
    dx = dg = db = None
    if backward:
        dy = to_device(inp.dy, wl, device)
        dx = dy if dx_over_dy else torch.empty_like(dy)
        dgt = torch.empty(C, device=device)
        dbt = torch.empty(C, device=device)
        iabn.iabn_backward(x, dy, dx, N, C, H, W, wl.layout, g, b, si, dgt, dbt, wl.act,
                           wl.act_param, ws)
        dg, db = dgt.cpu().numpy(), dbt.cpu().numpy()
    torch.cuda.synchronize()
    # no exchanging kernel gave up waiting for a partner (reads and clears the word)
    assert not iabn.iabn_workspace_status(ws), "exchange timeout recorded in the workspace"
    return GpuRun(y=x, dx=dx, save_mean=sm.cpu().numpy(), save_invstd=si.cpu().numpy(),
                  running_mean=rm.cpu().numpy(), running_var=rv.cpu().numpy(), dgamma=dg,
                  dbeta=db)


def check_forward(inp: workloads.Inputs, run: GpuRun, channels=None) -> dict:
    """Forward errors against the oracle on the same x bits (optionally a channel subset)."""
    wl = inp.wl
    x = storage_channels(inp.x, wl, channels)
    y = to_nchw64(run.y, wl, channels)
    sel = slice(None) if channels is None else np.asarray(_channel_index(channels, wl.C))
    f = oracle.forward_train(x, inp.gamma[sel], inp.beta[sel], wl.act, f32(wl.act_param),
                             f32(wl.eps), f32(wl.momentum), inp.running_mean[sel],
                             inp.running_var[sel], storage=wl.dtype)
    del x
    return {
        "y": rel_err_tensor(y, f["y"]),
        "save_mean": rel_err_vec(run.save_mean[sel], f["mean"]),
        "save_invstd": rel_err_vec(run.save_invstd[sel], f["invstd"]),
        "running_mean": rel_err_vec(run.running_mean[sel], f["running_mean"]),
        "running_var": rel_err_vec(run.running_var[sel], f["running_var"]),
    }


def _slope_from_y(y: np.ndarray, act: str, a: float) -> np.ndarray:
    if act == "leaky_relu":
        return np.where(y > 0, 1.0, a)
    if act == "elu":
        return np.where(y > 0, 1.0, y + a)
    return np.ones_like(y)


def check_backward(inp: workloads.Inputs, run: GpuRun, channels=None,
                   dx_scale: str = "rms") -> dict:
    """Backward errors against the oracle fed the GPU's own y bits and save_invstd.

    dx_scale="rms" (the gate everywhere): |g - o| / (|o| + rms_c(o)).
    dx_scale="terms": the denominator uses rms_c(gamma*invstd*dz), the size of the
    terms whose difference dx is.  Only for cases where dx is a near-total
    cancellation of those terms (m = 2: xhat^2 = v/(v+eps) ~ 1), where no fp32
    evaluation can carry relative accuracy in dx itself."""
    wl = inp.wl
    y = to_nchw64(run.y, wl, channels)
    dy = storage_channels(inp.dy, wl, channels)
    dx = to_nchw64(run.dx, wl, channels)
    sel = slice(None) if channels is None else np.asarray(_channel_index(channels, wl.C))
    o = oracle.backward_from_y(y, dy, inp.gamma[sel], inp.beta[sel],
                               run.save_invstd[sel].astype(np.float64), wl.act, f32(wl.act_param))
    if dx_scale == "terms":
        A = (inp.gamma[sel].astype(np.float64) * run.save_invstd[sel])[None, :, None, None]
        dz = _slope_from_y(y, wl.act, f32(wl.act_param)) * dy
        terms = np.sqrt(np.mean((A * dz) ** 2, axis=(0, 2, 3), keepdims=True))
        e_dx = float(np.max(np.abs(dx - o["dx"]) / (np.abs(o["dx"]) + terms + 1e-300)))
    else:
        e_dx = rel_err_tensor(dx, o["dx"])
    return {
        "dx": e_dx,
        "dgamma": rel_err_vec(run.dgamma[sel], o["dgamma"]),
        "dbeta": rel_err_vec(run.dbeta[sel], o["dbeta"]),
    }


def check_all_channels(inp: workloads.Inputs, run: GpuRun, block: int) -> dict:
    """Forward and backward errors over every element and channel, `block` channels
    at a time (bounds host memory on large tensors).  y and dx errors use each
    channel's own RMS as in check_forward / check_backward; the per-channel vectors
    are gathered over all C channels first and compared with the RMS over all C."""
    wl = inp.wl
    a = f32(wl.act_param)
    err = {"y": 0.0, "dx": 0.0}
    ref = {k: [] for k in ("mean", "invstd", "running_mean", "running_var", "dgamma", "dbeta")}
    for c0 in range(0, wl.C, block):
        sel = slice(c0, min(wl.C, c0 + block))
        x = storage_channels(inp.x, wl, sel)
        f = oracle.forward_train(x, inp.gamma[sel], inp.beta[sel], wl.act, a, f32(wl.eps),
                                 f32(wl.momentum), inp.running_mean[sel], inp.running_var[sel],
                                 storage=wl.dtype)
        del x
        y = to_nchw64(run.y, wl, sel)
        err["y"] = max(err["y"], rel_err_tensor(y, f["y"]))
        dy = storage_channels(inp.dy, wl, sel)
        o = oracle.backward_from_y(y, dy, inp.gamma[sel], inp.beta[sel],
                                   run.save_invstd[sel].astype(np.float64), wl.act, a)
        del y, dy
        err["dx"] = max(err["dx"], rel_err_tensor(to_nchw64(run.dx, wl, sel), o["dx"]))
        for k in ("mean", "invstd", "running_mean", "running_var"):
            ref[k].append(f[k])
        ref["dgamma"].append(o["dgamma"])
        ref["dbeta"].append(o["dbeta"])
    ref = {k: np.concatenate(v) for k, v in ref.items()}
    err["save_mean"] = rel_err_vec(run.save_mean, ref["mean"])
    err["save_invstd"] = rel_err_vec(run.save_invstd, ref["invstd"])
    err["running_mean"] = rel_err_vec(run.running_mean, ref["running_mean"])
    err["running_var"] = rel_err_vec(run.running_var, ref["running_var"])
    err["dgamma"] = rel_err_vec(run.dgamma, ref["dgamma"])
    err["dbeta"] = rel_err_vec(run.dbeta, ref["dbeta"])
    return err


def assert_within(errs: dict, dtype: str, what: str = "") -> None:
    tol = TOL[dtype]
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, "%s errors above %g: %s (all: %s)" % (what, tol, bad, errs)

"""GPU parity of optimized checkpointing (the block keeps xhat) against the fp64
oracle, through the C ABI.

Forward: GPU xhat (written over x) and statistics against the oracle on the
same x bits; y, which the forward forms from the stored xhat, against the
oracle's recompute from the GPU's own xhat bits.  Recompute: from the GPU's
xhat bits, bit-identical to the forward's y and within tolerance of the
oracle.  Backward: GPU dx, dgamma, dbeta against the oracle fed the GPU's own
xhat bits and save_invstd.  Gates as in tests/harness.py."""
import dataclasses

import numpy as np
import pytest
import torch

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import place_batchnorm_activation_amd as iabn


def custom(base, N, C, H, W, **kw):
    wl = workloads.config(base).with_shape(N, C, H, W)
    name = "%s_%dx%dx%dx%d" % (wl.name, N, C, H, W)
    for k, v in kw.items():
        name += "_%s=%s" % (k, v)
    return dataclasses.replace(wl, name=name, **kw)


def run_ckpt(inp, dx_over_dy=False):
    wl = inp.wl
    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    x = harness.to_device(inp.x, wl)
    y = torch.empty_like(x)
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    rm = torch.from_numpy(inp.running_mean).cuda()
    rv = torch.from_numpy(inp.running_var).cuda()
    sm, si = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(N, C, H, W, wl.layout, x.dtype)
    iabn.iabn_forward_train_ckpt(x, y, N, C, H, W, wl.layout, g, b, rm, rv, sm, si, wl.act,
                                 wl.act_param, wl.eps, wl.momentum, ws)
    yr = torch.empty_like(x)
    iabn.iabn_recompute_from_xhat(x, yr, N, C, H, W, wl.layout, g, b, wl.act, wl.act_param)
    dy = harness.to_device(inp.dy, wl)
    dx = dy if dx_over_dy else torch.empty_like(dy)
    dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    iabn.iabn_backward_ckpt(x, dy, dx, N, C, H, W, wl.layout, g, b, si, dg, db, wl.act,
                            wl.act_param, ws)
    torch.cuda.synchronize()
    return {"xhat": x, "y": y, "y_recomputed": yr, "dx": dx, "save_mean": sm.cpu().numpy(),
            "save_invstd": si.cpu().numpy(), "running_mean": rm.cpu().numpy(),
            "running_var": rv.cpu().numpy(), "dgamma": dg.cpu().numpy(),
            "dbeta": db.cpu().numpy()}


def check_ckpt(inp, r, block=None, dx_scale="rms"):
    """Errors over every element and channel, `block` channels at a time.
    dx_scale="terms": dx's error relative to the RMS of gamma*invstd*dz, the terms
    whose near-total cancellation dx is when m = 2 (as in harness.check_backward)."""
    wl = inp.wl
    a = harness.f32(wl.act_param)
    block = block or wl.C
    err = {"xhat": 0.0, "y": 0.0, "y_recomputed": 0.0, "dx": 0.0}
    info = {"y_from_x": 0.0}
    ref = {k: [] for k in ("mean", "invstd", "running_mean", "running_var", "dgamma", "dbeta")}
    for c0 in range(0, wl.C, block):
        sel = slice(c0, min(wl.C, c0 + block))
        x = harness.storage_channels(inp.x, wl, sel)
        f = oracle.forward_train_ckpt(x, inp.gamma[sel], inp.beta[sel], wl.act, a,
                                      harness.f32(wl.eps), harness.f32(wl.momentum),
                                      inp.running_mean[sel], inp.running_var[sel],
                                      storage=wl.dtype)
        del x
        xh = harness.to_nchw64(r["xhat"], wl, sel)
        err["xhat"] = max(err["xhat"], harness.rel_err_tensor(xh, f["xhat"]))
        # y is formed from the stored xhat (it equals the recompute), so it is gated
        # stage-wise, as a function of the GPU's xhat bits; the end-to-end error from
        # x, which adds xhat's storage rounding, is reported only
        yo = oracle.recompute_from_xhat(xh, inp.gamma[sel], inp.beta[sel], wl.act, a,
                                        storage=wl.dtype)
        gy = harness.to_nchw64(r["y"], wl, sel)
        err["y"] = max(err["y"], harness.rel_err_tensor(gy, yo))
        info["y_from_x"] = max(info["y_from_x"], harness.rel_err_tensor(gy, f["y"]))
        err["y_recomputed"] = max(err["y_recomputed"], harness.rel_err_tensor(
            harness.to_nchw64(r["y_recomputed"], wl, sel), yo))
        dy = harness.storage_channels(inp.dy, wl, sel)
        o = oracle.backward_from_xhat(xh, dy, inp.gamma[sel], inp.beta[sel],
                                      r["save_invstd"][sel].astype(np.float64), wl.act, a)
        gdx = harness.to_nchw64(r["dx"], wl, sel)
        if dx_scale == "terms":
            A = (inp.gamma[sel].astype(np.float64) * r["save_invstd"][sel])[None, :, None, None]
            z = inp.gamma[sel][None, :, None, None] * xh + inp.beta[sel][None, :, None, None]
            slope = {"leaky_relu": np.where(z > 0, 1.0, a),
                     "elu": np.where(z > 0, 1.0, a * np.exp(np.minimum(z, 0.0)))}.get(wl.act, 1.0)
            terms = np.sqrt(np.mean((A * slope * dy) ** 2, axis=(0, 2, 3), keepdims=True))
            e = float(np.max(np.abs(gdx - o["dx"]) / (np.abs(o["dx"]) + terms + 1e-300)))
        else:
            e = harness.rel_err_tensor(gdx, o["dx"])
        del dy
        err["dx"] = max(err["dx"], e)
        for k in ("mean", "invstd", "running_mean", "running_var"):
            ref[k].append(f[k])
        ref["dgamma"].append(o["dgamma"])
        ref["dbeta"].append(o["dbeta"])
    ref = {k: np.concatenate(v) for k, v in ref.items()}
    err["save_mean"] = harness.rel_err_vec(r["save_mean"], ref["mean"])
    err["save_invstd"] = harness.rel_err_vec(r["save_invstd"], ref["invstd"])
    err["running_mean"] = harness.rel_err_vec(r["running_mean"], ref["running_mean"])
    err["running_var"] = harness.rel_err_vec(r["running_var"], ref["running_var"])
    err["dgamma"] = harness.rel_err_vec(r["dgamma"], ref["dgamma"])
    err["dbeta"] = harness.rel_err_vec(r["dbeta"], ref["dbeta"])
    print("   not gated:", info, flush=True)
    return err


CASES = []
for layout in ("NCHW", "NHWC"):
    for dtype in ("f32", "bf16", "f16"):
        for act, p in (("leaky_relu", 0.01), ("elu", 1.0), ("identity", 0.0)):
            base = 4 if act == "elu" else (2 if dtype == "f32" else 3)
            # a vector-path shape and a ragged (single-element) one
            shapes = [(4, 16, 16, 20), (3, 5, 17, 19)] if layout == "NCHW" else \
                     [(3, 24, 9, 11), (2, 13, 10, 7)]
            for s in shapes:
                CASES.append(custom(base, *s, layout=layout, dtype=dtype, act=act, act_param=p))
CASES += [custom(4, 3, 7, 9, 9, act_param=0.5),                 # ELU alpha != 1
          custom(2, 2, 5, 1, 1),                                 # m = 2, the minimum
          custom(2, 3, 7, 8, 8, eps=0.0),
          custom(3, 2, 4104, 3, 3, dtype="bf16"),                 # many channels, short rows
          custom(2, 8, 64, 56, 56),                                # several tiles, NCHW fp32
          custom(3, 4, 256, 40, 60, layout="NHWC", dtype="bf16")]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_ckpt_matches_the_oracle(wl):
    inp = workloads.make_inputs(wl)
    print("case:", wl.name, wl.layout, wl.dtype, wl.act, wl.act_param, flush=True)
    r = run_ckpt(inp)
    # m = 2: dx is the eps/var-sized remainder of a cancellation (reading R15)
    err = check_ckpt(inp, r, dx_scale="terms" if wl.m == 2 else "rms")
    print("  ", err, flush=True)
    harness.assert_within(err, wl.dtype, wl.name)
    # the forward's y is formed from the stored xhat: the recompute gives its bits
    assert torch.equal(r["y"], r["y_recomputed"])


def test_ckpt_dx_in_place_and_deterministic():
    wl = custom(3, 4, 64, 16, 16, layout="NHWC", dtype="bf16")
    inp = workloads.make_inputs(wl)
    a, b = run_ckpt(inp), run_ckpt(inp, dx_over_dy=True)
    for k in ("xhat", "y", "dx"):
        assert torch.equal(a[k], b[k]), k
    for k in ("save_mean", "save_invstd", "running_mean", "running_var", "dgamma", "dbeta"):
        assert np.array_equal(a[k], b[k]), k


def test_ckpt_recompute_in_place():
    wl = custom(2, 2, 8, 6, 6)
    inp = workloads.make_inputs(wl)
    r = run_ckpt(inp)
    x = r["xhat"].clone()
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    iabn.iabn_recompute_from_xhat(x, x, wl.N, wl.C, wl.H, wl.W, wl.layout, g, b, wl.act,
                                  wl.act_param)
    torch.cuda.synchronize()
    assert torch.equal(x, r["y"])


@pytest.mark.parametrize("idx", [3, 2])
def test_ckpt_full_size_every_channel(idx):
    """The segmentation map and the ResNet mid-stage map at full size."""
    wl = workloads.config(idx)
    inp = workloads.make_inputs(wl)
    r = run_ckpt(inp)
    block = 32 if wl.storage_bytes > (128 << 20) else wl.C
    err = check_ckpt(inp, r, block)
    print("  ", wl.name, err, flush=True)
    harness.assert_within(err, wl.dtype, wl.name)
    assert torch.equal(r["y"], r["y_recomputed"])

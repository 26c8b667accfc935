"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Forward: GPU y / statistics / running statistics vs the oracle on the same x bits.
Backward: GPU dx / dgamma / dbeta vs the oracle on the GPU's own y bits and
save_invstd.  Gates: 1e-5 (fp32 storage) and 2e-2 (bf16 storage) on the
metric of tests/harness.py.
"""
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


def custom(base: int, N, C, H, W, **kw) -> workloads.Workload:
    wl = workloads.config(base).with_shape(N, C, H, W)
    name = "%s_%dx%dx%dx%d" % (wl.name, N, C, H, W)
    for k, v in kw.items():
        name += "_%s=%s" % (k, v)
    return dataclasses.replace(wl, name=name, **kw)


def full_check(wl, seed=None, channels=None, dx_over_dy=False):
    inp = workloads.make_inputs(wl, seed=seed)
    print("case:", wl.name, wl.layout, wl.dtype, wl.act, wl.act_param, flush=True)
    run = harness.run_gpu(inp, dx_over_dy=dx_over_dy)
    ef = harness.check_forward(inp, run, channels)
    # m = 2: dx is the eps/var-sized remainder of a cancellation (xhat = +-sqrt(v/(v+eps)));
    # its error is gated against the size of the cancelled terms instead
    eb = harness.check_backward(inp, run, channels, dx_scale="terms" if wl.m == 2 else "rms")
    print("  forward", ef, "\n  backward", eb, flush=True)
    harness.assert_within(ef, wl.dtype, "forward " + wl.name)
    harness.assert_within(eb, wl.dtype, "backward " + wl.name)
    return inp, run


# ---------------------------------------------------------------------------
# small and mid sizes: every layout x dtype x activation, several tiles, ragged tails

def test_config1_tiny():
    full_check(workloads.config(1))


MID = []
for layout in ("NCHW", "NHWC"):
    for dtype in ("f32", "bf16", "f16"):
        for act, p in (("leaky_relu", 0.01), ("elu", 1.0), ("identity", 0.0)):
            base = 4 if act == "elu" else (2 if dtype == "f32" else 3)
            # vector path shapes and scalar (ragged) path shapes
            if layout == "NCHW":
                shapes = [(4, 6, 16, 20), (3, 5, 17, 19)]
            else:
                # the first three fit the slice-resident kernels; the last has too
                # many rows for them and takes the split path
                shapes = [(3, 24, 9, 11), (2, 13, 10, 7), (2, 200, 12, 12), (2, 16, 80, 80)]
            for s in shapes:
                MID.append(custom(base, *s, layout=layout, dtype=dtype, act=act, act_param=p))


@pytest.mark.parametrize("wl", MID, ids=lambda w: w.name)
def test_mid_sizes(wl):
    full_check(wl)


# ---------------------------------------------------------------------------
# the five workloads at their full sizes, every element and channel against the
# oracle (the 268 MB segmentation map 32 channels at a time, to bound host memory)

@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_every_channel(idx):
    wl = workloads.config(idx)
    inp = workloads.make_inputs(wl)
    print("case:", wl.name, iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                                     workloads.storage_torch_dtype(wl.dtype),
                                                     wl.act), flush=True)
    run = harness.run_gpu(inp)
    block = 32 if wl.storage_bytes > (128 << 20) else wl.C
    errs = harness.check_all_channels(inp, run, block)
    print("  ", errs, flush=True)
    harness.assert_within(errs, wl.dtype, wl.name)
    # property that holds at any size: every channel's input gradient sums to zero
    dx = run.dx.float() if wl.layout == "NCHW" else run.dx.float().permute(0, 3, 1, 2)
    s = dx.sum(dim=(0, 2, 3)).double().cpu().numpy()
    a = dx.abs().sum(dim=(0, 2, 3)).double().cpu().numpy()
    tol = 1e-4 if wl.dtype == "f32" else 2e-2
    assert np.all(np.abs(s) <= tol * a + 1e-30), np.max(np.abs(s) / a)


# ---------------------------------------------------------------------------
# edge cases

EDGE = [
    custom(2, 2, 5, 1, 1),                                  # m = 2, the minimum
    custom(2, 1, 1, 300, 301),                               # one channel, long reduction
    custom(3, 2, 4104, 3, 3, dtype="bf16"),                  # many channels, short rows (NHWC)
    custom(2, 2, 4104, 3, 3, layout="NHWC"),                 # fp32 NHWC many channels
    custom(2, 3, 7, 8, 8, eps=0.0),                          # eps = 0
    custom(4, 3, 7, 9, 9, act_param=0.5),                    # ELU alpha != 1
    custom(2, 3, 7, 9, 9, act_param=1.0),                    # leaky slope 1 = identity
    custom(2, 3, 7, 9, 9, act_param=0.3, momentum=0.0),      # momentum 0
    custom(2, 3, 7, 9, 9, momentum=1.0),                     # momentum 1
    custom(2, 64, 3, 1, 1),                                  # tiny planes, many channels
    custom(5, 3, 8, 1, 1),                                   # NHWC with m = 3 rows
]


@pytest.mark.parametrize("wl", EDGE, ids=lambda w: w.name)
def test_edge_cases(wl):
    full_check(wl)


def test_constant_channel():
    wl = custom(2, 2, 3, 4, 4)
    inp = workloads.make_inputs(wl)
    inp.x[:, 1] = np.float32(2.5)        # variance 0 in channel 1: xhat = 0, y = act(beta)
    run = harness.run_gpu(inp)
    harness.assert_within(harness.check_forward(inp, run), "f32", "forward")
    harness.assert_within(harness.check_backward(inp, run), "f32", "backward")


@pytest.mark.parametrize("layout,dtype", [("NCHW", "f32"), ("NHWC", "bf16"), ("NCHW", "bf16"),
                                          ("NHWC", "f32")])
def test_misaligned_pointers_take_scalar_path(layout, dtype):
    """Tensors one element off 16-byte alignment: same results within tolerance."""
    wl = custom(2 if dtype == "f32" else 3, 2, 16, 8, 8, layout=layout, dtype=dtype)
    inp = workloads.make_inputs(wl)
    n = wl.numel
    tdt = workloads.storage_torch_dtype(dtype)
    bx = torch.empty(n + 1, dtype=tdt, device="cuda")
    bdy = torch.empty(n + 1, dtype=tdt, device="cuda")
    bdx = torch.empty(n + 1, dtype=tdt, device="cuda")
    x = bx[1:]
    x.copy_(workloads.to_torch(inp.x, dtype).reshape(-1))
    dy = bdy[1:]
    dy.copy_(workloads.to_torch(inp.dy, dtype).reshape(-1))
    dx = bdx[1:]
    assert x.data_ptr() % 16 != 0
    C = wl.C
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    sm, si = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(wl.N, C, wl.H, wl.W, layout, tdt)
    iabn.iabn_forward_train(x, wl.N, C, wl.H, wl.W, layout, g, b, None, None, sm, si, wl.act,
                            wl.act_param, wl.eps, wl.momentum, ws)
    iabn.iabn_backward(x, dy, dx, wl.N, C, wl.H, wl.W, layout, g, b, si, dg, db, wl.act,
                       wl.act_param, ws)
    torch.cuda.synchronize()
    run = harness.GpuRun(y=x.reshape(harness.storage_shape(wl)),
                         dx=dx.reshape(harness.storage_shape(wl)), save_mean=sm.cpu().numpy(),
                         save_invstd=si.cpu().numpy(), running_mean=inp.running_mean,
                         running_var=inp.running_var, dgamma=dg.cpu().numpy(),
                         dbeta=db.cpu().numpy())
    ef = harness.check_forward(inp, run)
    ef.pop("running_mean")
    ef.pop("running_var")
    harness.assert_within(ef, dtype, "forward")
    harness.assert_within(harness.check_backward(inp, run), dtype, "backward")


# ---------------------------------------------------------------------------
# determinism, aliasing, stage entry points, inference

@pytest.mark.parametrize("wl", [custom(2, 8, 32, 28, 28), custom(3, 4, 64, 32, 32),
                                custom(4, 4, 32, 14, 14), custom(5, 8, 512, 7, 7),
                                custom(3, 5, 256, 40, 60, layout="NHWC", dtype="bf16"),
                                custom(3, 1, 256, 300, 300, layout="NHWC", dtype="bf16"),
                                # the four full-size workloads in the kernels they plan:
                                # channel-resident NCHW, streamed slice forward + split
                                # backward, dy-resident NCHW ELU, eight-lane groups of 8
                                workloads.config(2), workloads.config(3), workloads.config(4),
                                workloads.config(5)],
                         ids=lambda w: w.name)
def test_bitwise_deterministic(wl):
    inp = workloads.make_inputs(wl)
    runs = [harness.run_gpu(inp) for _ in range(3)]
    for r in runs[1:]:
        assert torch.equal(r.y, runs[0].y)
        assert torch.equal(r.dx, runs[0].dx)
        for k in ("save_mean", "save_invstd", "running_mean", "running_var", "dgamma", "dbeta"):
            assert np.array_equal(getattr(r, k), getattr(runs[0], k)), k


@pytest.mark.parametrize("idx", [2, 3])
def test_dx_in_place_over_dy(idx):
    wl = workloads.config(idx).with_shape(4, 64, 16, 16)
    inp = workloads.make_inputs(wl)
    a = harness.run_gpu(inp)
    b = harness.run_gpu(inp, dx_over_dy=True)
    assert torch.equal(a.dx, b.dx)
    assert np.array_equal(a.dgamma, b.dgamma) and np.array_equal(a.dbeta, b.dbeta)


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_stage_entry_points(idx):
    """The stage entry points (always the split kernels) against the oracle and
    against iabn_forward_train / iabn_backward (which may take the
    channel-resident kernels: same values up to rounding order)."""
    wl = workloads.config(idx).with_shape(4, 32 if idx != 5 else 256, 12, 12)
    inp = workloads.make_inputs(wl)
    ref = harness.run_gpu(inp)
    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    x = harness.to_device(inp.x, wl)
    dy = harness.to_device(inp.dy, wl)
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    rm = torch.from_numpy(inp.running_mean).cuda()
    rv = torch.from_numpy(inp.running_var).cuda()
    sm, si = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    dx = torch.empty_like(dy)
    ws = iabn.workspace(N, C, H, W, wl.layout, x.dtype)
    x0 = x.clone()
    iabn.iabn_forward_stats(x, N, C, H, W, wl.layout, g, b, rm, rv, sm, si, wl.eps, wl.momentum,
                            ws)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)            # the statistics stage does not write x
    iabn.iabn_forward_apply(x, N, C, H, W, wl.layout, wl.act, wl.act_param, ws)
    y0 = x.clone()
    iabn.iabn_backward_reduce(x, dy, N, C, H, W, wl.layout, g, b, si, dg, db, wl.act,
                              wl.act_param, ws)
    iabn.iabn_backward_apply(x, dy, dx, N, C, H, W, wl.layout, wl.act, wl.act_param, ws)
    torch.cuda.synchronize()
    assert torch.equal(x, y0)            # the backward never writes y
    run = harness.GpuRun(y=x, dx=dx, save_mean=sm.cpu().numpy(), save_invstd=si.cpu().numpy(),
                         running_mean=rm.cpu().numpy(), running_var=rv.cpu().numpy(),
                         dgamma=dg.cpu().numpy(), dbeta=db.cpu().numpy())
    harness.assert_within(harness.check_forward(inp, run), wl.dtype, "stage forward")
    harness.assert_within(harness.check_backward(inp, run), wl.dtype, "stage backward")
    tol = harness.TOL[wl.dtype]
    assert harness.rel_err_tensor(harness.to_nchw64(x, wl), harness.to_nchw64(ref.y, wl)) <= tol
    assert harness.rel_err_vec(run.save_invstd, ref.save_invstd) <= tol
    assert harness.rel_err_vec(run.dgamma, ref.dgamma) <= tol
    if "split" in iabn.iabn_describe_plan(N, C, H, W, wl.layout, x.dtype, wl.act):
        assert torch.equal(x, ref.y) and torch.equal(dx, ref.dx)   # same kernels: same bits


# every channel-resident variant, picked through the channel length it holds
def _variant_shapes():
    out = []
    for dtype, V in (("f32", 4), ("bf16", 8)):
        for vc in (200, 400, 1000, 2000, 3300, 8000, 16000, 25000):
            m = vc * V                      # elements per channel: N=2, H=1, W=m/2
            base = 2 if dtype == "f32" else 3
            out.append(custom(base, 2, 3, 1, m // 2, layout="NCHW", dtype=dtype))
        for vc in (3300, 25000):
            out.append(custom(4, 2, 3, 1, vc * V // 2, layout="NCHW", dtype=dtype, act="elu",
                              act_param=1.0))
    for vc in (1000, 3300, 16000, 25000):                   # fp16: 8 elements per vector
        out.append(custom(3, 2, 3, 1, vc * 4, layout="NCHW", dtype="f16"))
    return out


# every channel-resident variant on single elements: 7x7 planes (not a multiple
# of the vector width) with N chosen so that m = 49*N just fits each capacity
# (512 ... 24576 elements), storage dtypes and activations mixed
def _scalar_shapes():
    out = []
    caps = [(10, "f32"), (20, "bf16"), (41, "f16"), (83, "f32"), (167, "bf16"), (334, "f32"),
            (501, "f16")]
    for k, (N, dtype) in enumerate(caps):
        base = 2 if dtype == "f32" else 3
        act = ("leaky_relu", "elu", "identity")[k % 3]
        p = {"leaky_relu": 0.01, "elu": 1.0, "identity": 0.0}[act]
        out.append(custom(base, N, 3, 7, 7, layout="NCHW", dtype=dtype, act=act, act_param=p))
    out.append(custom(2, 32, 256, 7, 7))                       # an NCHW 7x7 tail, fp32
    return out


@pytest.mark.parametrize("wl", _scalar_shapes(), ids=lambda w: w.name)
def test_channel_resident_scalar_variants(wl):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    print(desc)
    assert "channel_resident_scalar" in desc
    full_check(wl)


# Tensors beyond 4 GiB: the resident kernels address with 32-bit offsets and must
# step aside; the split kernels index with 64 bits.  Inputs are drawn on the
# device; the oracle checks sampled channels (first, middle, last).
BIG = [custom(2, 8, 16, 2048, 4100),                              # fp32 NCHW, 4.3 GB
       custom(3, 4, 512, 1024, 1025, layout="NHWC", dtype="bf16")]   # bf16 NHWC, 4.3 GB


@pytest.mark.parametrize("wl", BIG, ids=lambda w: w.name)
def test_beyond_4gib(wl):
    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    assert wl.storage_bytes > 2 ** 32
    desc = iabn.iabn_describe_plan(N, C, H, W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    assert desc.startswith("forward=split") and "backward=split" in desc, desc
    inp = workloads.make_device_inputs(wl, seed=4242)
    chans = [0, C // 2, C - 1]
    x_ch = [workloads.device_channel(inp.x, wl, c) for c in chans]
    dy_ch = [workloads.device_channel(inp.dy, wl, c) for c in chans]
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    rm = torch.from_numpy(inp.running_mean).cuda()
    rv = torch.from_numpy(inp.running_var).cuda()
    sm, si = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(N, C, H, W, wl.layout, inp.x.dtype)
    print("case:", wl.name, desc, flush=True)
    iabn.iabn_forward_train(inp.x, N, C, H, W, wl.layout, g, b, rm, rv, sm, si, wl.act,
                            wl.act_param, wl.eps, wl.momentum, ws)
    iabn.iabn_backward(inp.x, inp.dy, inp.dy, N, C, H, W, wl.layout, g, b, si, dg, db, wl.act,
                       wl.act_param, ws)           # dx over dy
    torch.cuda.synchronize()
    sm, si, dg, db = (t.cpu().numpy() for t in (sm, si, dg, db))
    ref = {k: [] for k in ("mean", "invstd", "dgamma", "dbeta")}
    errs = {"y": 0.0, "dx": 0.0}
    for k, c in enumerate(chans):
        f = oracle.forward_train(x_ch[k], inp.gamma[c:c + 1], inp.beta[c:c + 1], wl.act,
                                 harness.f32(wl.act_param), harness.f32(wl.eps),
                                 storage=wl.dtype)
        y_gpu = workloads.device_channel(inp.x, wl, c)
        errs["y"] = max(errs["y"], harness.rel_err_tensor(y_gpu, f["y"]))
        o = oracle.backward_from_y(y_gpu, dy_ch[k], inp.gamma[c:c + 1], inp.beta[c:c + 1],
                                   si[c:c + 1].astype(np.float64), wl.act,
                                   harness.f32(wl.act_param))
        del y_gpu
        dx_gpu = workloads.device_channel(inp.dy, wl, c)
        errs["dx"] = max(errs["dx"], harness.rel_err_tensor(dx_gpu, o["dx"]))
        for key, src in (("mean", f), ("invstd", f), ("dgamma", o), ("dbeta", o)):
            ref[key].append(src[key][0])
    errs["save_mean"] = harness.rel_err_vec(sm[chans], np.array(ref["mean"]))
    errs["save_invstd"] = harness.rel_err_vec(si[chans], np.array(ref["invstd"]))
    errs["dgamma"] = harness.rel_err_vec(dg[chans], np.array(ref["dgamma"]))
    errs["dbeta"] = harness.rel_err_vec(db[chans], np.array(ref["dbeta"]))
    print("  channels", chans, errs, flush=True)
    harness.assert_within(errs, wl.dtype, wl.name)


# every slice-resident NHWC variant and group sizes 1 to 16, picked through the
# row count and slice count (the plan is asserted): full and ragged members;
# slice counts that divide by 8 (XCD-grouped map) and ones that do not
SLICE_PLANS = [
    # one lane per row, 256 threads: tensors under 4 MB (at most 2, else 4 rows
    # per thread, groups up to 8) and odd vector counts per row
    (custom(2, 1, 8, 7, 7, layout="NHWC", dtype="f32"), "256x1x2"),
    (custom(2, 2, 20, 7, 9, layout="NHWC", dtype="f32"), "256x1x2"),
    (custom(2, 1, 64, 40, 13, layout="NHWC", dtype="f32"), "256x1x2,group2"),
    (custom(3, 1, 64, 80, 13, layout="NHWC", dtype="f16"), "256x1x2,group4"),
    (custom(2, 2, 64, 80, 13, layout="NHWC", dtype="f32"), "256x1x2,group8"),
    (custom(2, 1, 8, 40, 13, layout="NHWC", dtype="f32"), "256x1x4"),
    (custom(2, 1, 384, 80, 13, layout="NHWC", dtype="f32"), "256x1x4,group2"),
    (custom(2, 2, 192, 80, 13, layout="NHWC", dtype="f32"), "256x1x4,group4"),
    (custom(2, 5, 64, 25, 33, layout="NHWC", dtype="f32"), "256x1x4,group8"),
    (custom(3, 32, 256, 14, 14, layout="NHWC", dtype="bf16"), "256x1x4,group8"),
    (custom(3, 1, 8, 80, 13, layout="NHWC", dtype="bf16"), "256x1x8"),
    (custom(2, 5, 44, 20, 20, layout="NHWC", dtype="f32"), "256x1x8"),
    (custom(3, 2, 8, 80, 13, layout="NHWC", dtype="bf16"), "256x1x13"),
    (custom(3, 4, 200, 25, 33, layout="NHWC", dtype="bf16"), "256x1x13"),
    # one lane per row, 512 threads
    (custom(3, 6, 8, 7, 80, layout="NHWC", dtype="bf16"), "512x1x13"),
    (custom(5, 3, 1032, 40, 50, layout="NHWC", dtype="bf16"), "512x1x13"),
    (custom(2, 5, 520, 80, 17, layout="NHWC", dtype="f32"), "512x1x18"),
    # two lanes per row
    (custom(2, 1, 1032, 60, 17, layout="NHWC", dtype="f32"), "512x2x4"),
    (custom(2, 5, 192, 25, 33, layout="NHWC", dtype="f32"), "512x2x4,group8"),
    (custom(2, 5, 64, 33, 50, layout="NHWC", dtype="f32"), "512x2x4,group16"),
    # ResNet-50 maps where two lanes in half the group replace four lanes in
    # the two-level exchange
    (custom(3, 8, 512, 28, 28, layout="NHWC", dtype="bf16"), "512x2x4,group8"),
    (custom(3, 64, 256, 14, 14, layout="NHWC", dtype="bf16"), "512x2x4,group16"),
    (custom(2, 8, 64, 33, 64, layout="NHWC", dtype="f32"), "512x2x4,group32"),
    (custom(2, 1, 8, 80, 13, layout="NHWC", dtype="f32"), "512x2x8"),
    (custom(2, 1, 768, 60, 60, layout="NHWC", dtype="f32"), "512x2x8,group2"),
    (custom(2, 2, 384, 60, 60, layout="NHWC", dtype="f32"), "512x2x8,group4"),
    (custom(2, 5, 192, 33, 50, layout="NHWC", dtype="f32"), "512x2x8,group8"),
    (custom(2, 6, 128, 60, 80, layout="NHWC", dtype="f32"), "512x2x8,group16"),
    (custom(2, 6, 64, 80, 80, layout="NHWC", dtype="f32"), "512x2x8,group32"),
    (custom(2, 2, 8, 80, 13, layout="NHWC", dtype="f32"), "512x2x13"),
    (custom(2, 8, 192, 33, 64, layout="NHWC", dtype="f32"), "512x2x13,group8"),
    (custom(2, 6, 8, 7, 80, layout="NHWC", dtype="f32"), "512x2x18"),
    # four lanes per row
    (custom(2, 1, 2064, 30, 17, layout="NHWC", dtype="f32"), "512x4x4"),
    (custom(2, 3, 1536, 7, 33, layout="NHWC", dtype="f32"), "512x4x4,group2"),
    (custom(2, 1, 768, 80, 13, layout="NHWC", dtype="f32"), "512x4x4,group4"),
    (custom(2, 2, 384, 80, 13, layout="NHWC", dtype="f32"), "512x4x4,group8"),
    (custom(2, 5, 256, 25, 33, layout="NHWC", dtype="f32"), "512x2x4,group8"),
    (custom(2, 5, 128, 33, 50, layout="NHWC", dtype="f32"), "512x2x4,group16"),
    (custom(2, 1, 1152, 13, 80, layout="NHWC", dtype="f32"), "512x4x7,group2"),
    (custom(2, 2, 640, 13, 80, layout="NHWC", dtype="f32"), "512x4x7,group4"),
    (custom(2, 5, 384, 25, 33, layout="NHWC", dtype="f32"), "512x4x7,group8"),
    (custom(2, 5, 256, 33, 50, layout="NHWC", dtype="f32"), "512x4x7,group16"),
    (custom(2, 8, 128, 33, 64, layout="NHWC", dtype="f32"), "512x4x7,group32"),
    (custom(2, 2, 1152, 13, 80, layout="NHWC", dtype="f32"), "512x4x13,group2"),
    (custom(2, 5, 640, 25, 33, layout="NHWC", dtype="f32"), "512x4x13,group4"),
    (custom(2, 5, 384, 33, 50, layout="NHWC", dtype="f32"), "512x4x13,group8"),
    (custom(2, 8, 256, 33, 64, layout="NHWC", dtype="f32"), "512x4x13,group16"),
    (custom(3, 5, 512, 50, 80, layout="NHWC", dtype="bf16"), "512x4x13,group16"),
    (custom(2, 6, 128, 80, 80, layout="NHWC", dtype="f32"), "512x4x13,group32"),
    # eight lanes per row (whole lines), 7 or 13 rows a thread, groups of at most 8
    (custom(2, 1, 1280, 13, 80, layout="NHWC", dtype="f32"), "512x8x7,group4"),
    (custom(5, 64, 2048, 7, 7, layout="NHWC", dtype="bf16"), "512x8x7,group8"),
    (custom(2, 2, 1280, 13, 80, layout="NHWC", dtype="f32"), "512x8x13,group4"),
    (custom(2, 5, 768, 25, 33, layout="NHWC", dtype="f32"), "512x8x13,group8"),
    (custom(3, 5, 2048, 30, 30, layout="NHWC", dtype="bf16"), "512x8x13,group8"),
    # other storage types and activations
    (custom(3, 8, 2048, 10, 25, layout="NHWC", dtype="f16"), "512x4x4,group4"),
    (custom(5, 8, 2048, 10, 25, layout="NHWC", dtype="f16", act="elu", act_param=1.0),
     "512x4x4,group4"),
    (custom(4, 5, 768, 25, 33, layout="NHWC", dtype="f32", act="elu", act_param=1.0),
     "512x8x13,group8"),
    (custom(4, 5, 256, 25, 33, layout="NHWC", dtype="f32", act="elu", act_param=1.0),
     "512x2x4,group8"),
    (custom(4, 3, 512, 12, 12, layout="NHWC", dtype="bf16", act="elu", act_param=0.5),
     "256x1x2"),
    (custom(3, 5, 256, 20, 20, layout="NHWC", dtype="bf16", act="identity", act_param=0.0),
     "256x1x2,group4"),
    (custom(2, 2, 256, 60, 60, layout="NHWC", dtype="f32", act="identity", act_param=0.0),
     "512x2x4,group8"),
]


def _slice_shapes():
    return [wl for wl, _ in SLICE_PLANS]


@pytest.mark.parametrize("wl,plan", SLICE_PLANS, ids=[w.name for w, _ in SLICE_PLANS])
def test_slice_resident_plans(wl, plan):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    assert desc == "forward=slice_resident(%s) backward=slice_resident(%s)" % (plan, plan)


@pytest.mark.parametrize("wl", _slice_shapes(), ids=lambda w: w.name)
def test_slice_resident_variants(wl):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    print(desc)
    assert "slice_resident" in desc
    full_check(wl)


# NCHW channels shared by groups of workgroups (channels one workgroup cannot
# hold, or too few to fill the chip): every group size from 2 to 64, ragged
# shares, the two-level exchange from 16 members, every storage type and
# activation.  (case, forward plan, backward plan)
CHANNEL_GROUPS = [
    (custom(2, 3, 64, 97, 100), "512x16,group2", "512x16,dy_streamed,group2"),
    (custom(3, 8, 64, 80, 84, layout="NCHW", dtype="bf16"), "512x16,group2", "512x16,dy_streamed,group2"),
    (custom(2, 4, 5, 160, 160), "512x16,group4", "512x16,dy_streamed,group4"),
    (custom(3, 3, 48, 300, 300, layout="NCHW", dtype="bf16"), "512x32,group4", "512x32,dy_streamed,group4"),
    (custom(4, 3, 24, 300, 300, act="elu", act_param=1.0), "512x32,group8",
     "512x32,dy_streamed,group8"),
    (custom(3, 3, 2, 300, 300, layout="NCHW", dtype="f16"), "512x16,group8", "512x16,dy_streamed,group8"),
    (custom(2, 3, 2, 300, 300, act="identity", act_param=0.0), "512x16,group16",
     "512x16,dy_streamed,group16"),
    (custom(2, 5, 2, 300, 300), "512x16,group32", "512x16,dy_streamed,group32"),
    (custom(3, 32, 1, 200, 200, layout="NCHW", dtype="bf16"), "512x16,group32", "512x16,dy_streamed,group32"),
    (custom(2, 32, 2, 200, 200), "512x16,group64", "512x16,dy_streamed,group64"),
    (custom(2, 32, 64, 112, 112), "512x49,group4", "512x49,dy_streamed,group4"),
    (custom(4, 32, 64, 112, 112, act="elu", act_param=1.0), "512x49,group4",
     "512x49,dy_streamed,group4"),
]


@pytest.mark.parametrize("wl,fwd,bwd", CHANNEL_GROUPS, ids=[w.name for w, _, _ in CHANNEL_GROUPS])
def test_channel_groups(wl, fwd, bwd):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    assert desc == "forward=channel_resident(%s) backward=channel_resident(%s)" % (fwd, bwd), desc
    full_check(wl)


def test_channel_groups_ignore_workspace_contents():
    """A grouped NCHW plan gives the same bits with a workspace of arbitrary
    contents, twice in a row on one workspace, and with dx over dy."""
    wl = custom(3, 3, 48, 300, 300, layout="NCHW", dtype="bf16")
    inp = workloads.make_inputs(wl)
    first = harness.run_gpu(inp)
    ws = iabn.workspace(wl.N, wl.C, wl.H, wl.W, wl.layout, first.y.dtype)
    ws.random_(0, 256)
    _same_run(harness.run_gpu(inp, ws=ws), first)
    _same_run(harness.run_gpu(inp, ws=ws), first)
    _same_run(harness.run_gpu(inp, dx_over_dy=True, ws=ws), first)


# NHWC maps the slice kernels cannot take (eight channel vectors a row): the
# split kernels' two-stage pipelines run several sets a thread.  2x64x300x300
# bf16: 5 sets of row groups per statistics / sums workgroup and 2 sets of dx
# vectors per thread, with remainders; 1x32x480x430 fp32: 6 sets and 3.
SPLIT_PIPELINE = [custom(3, 2, 64, 300, 300, layout="NHWC", dtype="bf16"),
                  custom(2, 1, 32, 480, 430, layout="NHWC", dtype="f32", act="identity",
                         act_param=0.0)]


@pytest.mark.parametrize("wl", SPLIT_PIPELINE, ids=lambda w: w.name)
def test_split_pipelines(wl):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    assert desc == ("forward=split(stats:256x256,apply:512x256,vec16) "
                    "backward=split(reduce:256x256,apply:512x256,vec16)"), desc
    full_check(wl)


# Streamed slice kernels (NHWC maps too large to hold): 256 workgroups, groups
# of 8 to 64, eight lanes per row (four where 16 vectors make a pixel).  Threads
# keep 28 rows in registers and 16 in LDS (forward: four chunks of 4) or 14 and
# 8 (backward: four chunks of 2) and stream the rest.  The backward streams only
# while at least half its rows stay on chip (else the split kernels).  The cases
# cover, in each direction, no chunk past the registers, one to four chunks kept
# in LDS only, and one to six chunks streamed past them (forward 1-6; backward
# 1-6, 8, 9 and 11), odd and even.
# after a streamed forward the dx pass runs one workgroup per CU (two elsewhere)
_SPLIT_BWD = "split(reduce:256x256,apply:256x256,vec16)"
_SPLIT_BWD_ELU = "split(reduce:256x256,apply:2048x256,vec16)"   # ELU: a wider dx grid
STREAM_PLANS = [
    (custom(3, 1, 256, 340, 340, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(3, 1, 256, 390, 390, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(2, 1, 128, 400, 400, layout="NHWC", dtype="f32"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(2, 1, 128, 436, 436, layout="NHWC", dtype="f32"),
     "slice_streamed(512x8x(28+16)+4,group64)", _SPLIT_BWD),
    (custom(3, 1, 128, 360, 360, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x4x(28+16)+4,group64)", "slice_streamed(512x4x(14+8)+2,group64)"),
    (custom(4, 1, 1024, 180, 170, layout="NHWC", dtype="f16", act="elu", act_param=1.0),
     "slice_streamed(512x8x(28+16)+4,group16)", "slice_streamed(512x8x(14+8)+2,group16)"),
    (custom(4, 1, 64, 600, 600, layout="NHWC", dtype="f32", act="elu", act_param=1.0),
     "slice_streamed(512x4x(28+16)+4,group64)", "slice_streamed(512x4x(14+8)+2,group64)"),
    (custom(3, 1, 256, 300, 300, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(2, 1, 128, 300, 310, layout="NHWC", dtype="f32"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(4, 1, 1024, 130, 130, layout="NHWC", dtype="f16", act="elu", act_param=1.0),
     "slice_streamed(512x8x(28+16)+4,group16)", "slice_streamed(512x8x(14+8)+2,group16)"),
    (custom(3, 3, 512, 100, 100, layout="NHWC", dtype="bf16", act="identity", act_param=0.0),
     "slice_streamed(512x8x(28+16)+4,group32)", "slice_streamed(512x8x(14+8)+2,group32)"),
    (custom(3, 1, 2048, 100, 100, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group8)", "slice_streamed(512x8x(14+8)+2,group8)"),
    # forward two chunks in LDS, backward six past them
    (custom(3, 1, 256, 362, 364, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    # backward two, three and five chunks past LDS
    (custom(3, 1, 256, 314, 316, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(4, 2, 256, 232, 233, layout="NHWC", dtype="f16", act="elu", act_param=1.0),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    (custom(2, 2, 128, 248, 249, layout="NHWC", dtype="f32"),
     "slice_streamed(512x8x(28+16)+4,group64)", "slice_streamed(512x8x(14+8)+2,group64)"),
    # forward two to six chunks past LDS
    (custom(4, 2, 512, 222, 223, layout="NHWC", dtype="f16", act="elu", act_param=1.0),
     "slice_streamed(512x8x(28+16)+4,group32)", _SPLIT_BWD_ELU),
    (custom(2, 2, 128, 326, 327, layout="NHWC", dtype="f32"),
     "slice_streamed(512x8x(28+16)+4,group64)", _SPLIT_BWD),
    (custom(3, 2, 256, 340, 341, layout="NHWC", dtype="f16"),
     "slice_streamed(512x8x(28+16)+4,group64)", _SPLIT_BWD),
    (custom(3, 1, 256, 496, 498, layout="NHWC", dtype="bf16"),
     "slice_streamed(512x8x(28+16)+4,group64)", _SPLIT_BWD),
    (custom(2, 2, 128, 362, 363, layout="NHWC", dtype="f32"),
     "slice_streamed(512x8x(28+16)+4,group64)", _SPLIT_BWD),
]


@pytest.mark.parametrize("wl,fwd,bwd", STREAM_PLANS, ids=[w.name for w, _, _ in STREAM_PLANS])
def test_slice_streamed(wl, fwd, bwd):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    assert desc == "forward=%s backward=%s" % (fwd, bwd)
    full_check(wl)


def test_streamed_dx_in_place_and_fresh_workspace():
    """The streamed kernels (forward streaming, backward streaming) give the same
    bits with dx written over dy and with a workspace of arbitrary contents."""
    wl = custom(3, 1, 256, 300, 300, layout="NHWC", dtype="bf16")
    inp = workloads.make_inputs(wl)
    a = harness.run_gpu(inp)
    b = harness.run_gpu(inp, dx_over_dy=True)
    assert torch.equal(a.y, b.y) and torch.equal(a.dx, b.dx)
    ws = iabn.workspace(wl.N, wl.C, wl.H, wl.W, wl.layout, a.y.dtype)
    ws.random_(0, 256)
    c = harness.run_gpu(inp, ws=ws)
    assert torch.equal(a.y, c.y) and torch.equal(a.dx, c.dx)
    assert np.array_equal(a.dgamma, c.dgamma) and np.array_equal(a.save_invstd, c.save_invstd)


def _same_run(r, q):
    assert torch.equal(r.y, q.y) and torch.equal(r.dx, q.dx)
    for k in ("save_mean", "save_invstd", "running_mean", "running_var", "dgamma", "dbeta"):
        assert np.array_equal(getattr(r, k), getattr(q, k)), k


def test_group_exchange_ignores_workspace_contents():
    """Groups of workgroups swap partial sums through the workspace in words tagged
    with a token of the call (a per-slice epoch that the kernels advance): the
    results must not depend on what the workspace held -- a fill of ones, zeros or
    random bytes, another shape's exchange, or the same shape's previous call."""
    a = custom(3, 4, 256, 25, 33, layout="NHWC", dtype="bf16")      # group 4
    b = custom(3, 5, 256, 40, 60, layout="NHWC", dtype="bf16")      # group 16, two levels
    dt = workloads.storage_torch_dtype("bf16")
    size = max(iabn.iabn_workspace_size(w.N, w.C, w.H, w.W, w.layout, dt) for w in (a, b))
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    ina, inb = workloads.make_inputs(a), workloads.make_inputs(b)
    ws.fill_(0xFF)
    first = harness.run_gpu(ina, ws=ws)
    harness.assert_within(harness.check_forward(ina, first), "bf16", "forward")
    harness.assert_within(harness.check_backward(ina, first), "bf16", "backward")
    rb = harness.run_gpu(inb, ws=ws)
    harness.assert_within(harness.check_forward(inb, rb), "bf16", "forward")
    harness.assert_within(harness.check_backward(inb, rb), "bf16", "backward")
    _same_run(harness.run_gpu(ina, ws=ws), first)
    ws.zero_()
    _same_run(harness.run_gpu(ina, ws=ws), first)
    ws.random_(0, 256)
    _same_run(harness.run_gpu(ina, ws=ws), first)
    for _ in range(3):
        _same_run(harness.run_gpu(ina, ws=ws), first)
    _same_run(harness.run_gpu(ina, dx_over_dy=True, ws=ws), first)


# Channels whose first element -- the pivot of the shifted sums -- lies 8 standard
# deviations from the mean (alternating sides): the statistics must not lose
# accuracy to the shift.  One case per kernel family.
OUTLIER = [custom(2, 4, 32, 16, 16),                                   # NCHW channel-resident
           custom(2, 3, 5, 17, 19),                                    # NCHW resident, elements
           custom(2, 1, 3, 157, 163),                                  # NCHW split, scalar
           custom(3, 4, 256, 25, 33, layout="NHWC", dtype="bf16"),     # NHWC slice-resident
           custom(2, 4, 96, 25, 33, layout="NHWC", dtype="f32"),       # (groups of 4)
           custom(3, 5, 2048, 30, 30, layout="NHWC", dtype="bf16"),    # 8 lanes, group 8
           custom(2, 5, 640, 25, 33, layout="NHWC", dtype="f32"),      # 4 lanes, group 4
           custom(2, 8, 256, 33, 64, layout="NHWC", dtype="f32"),      # group 16, two levels
           custom(3, 1, 256, 340, 340, layout="NHWC", dtype="bf16"),   # streamed, 8 lanes
           custom(3, 1, 128, 360, 360, layout="NHWC", dtype="bf16"),   # streamed, 4 lanes
           # fp32 streamed slices under the 1e-5 gate: about 78 (8 lanes, groups of
           # 64) and 20 (4 lanes) rows summed per thread
           custom(2, 2, 128, 400, 400, layout="NHWC", dtype="f32"),
           custom(2, 1, 64, 400, 400, layout="NHWC", dtype="f32"),
           custom(2, 2, 16, 80, 80, layout="NHWC", dtype="f32")]       # NHWC split


@pytest.mark.parametrize("wl", OUTLIER, ids=lambda w: w.name)
def test_outlier_pivot(wl):
    inp = workloads.make_inputs(wl)
    x = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    mu, sd = x.mean(axis=(0, 2, 3)), x.std(axis=(0, 2, 3))
    side = np.where(np.arange(wl.C) % 2 == 0, 1.0, -1.0)
    x[0, :, 0, 0] = mu + side * 8.0 * sd
    inp = dataclasses.replace(inp, x=workloads.to_storage(x, wl.layout, wl.dtype))
    print("case:", wl.name, "outlier pivots", flush=True)
    run = harness.run_gpu(inp)
    ef = harness.check_forward(inp, run)
    eb = harness.check_backward(inp, run)
    print("  forward", ef, "\n  backward", eb, flush=True)
    harness.assert_within(ef, wl.dtype, "forward " + wl.name)
    harness.assert_within(eb, wl.dtype, "backward " + wl.name)


@pytest.mark.parametrize("wl", _variant_shapes(), ids=lambda w: w.name)
def test_channel_resident_variants(wl):
    desc = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout,
                                   workloads.storage_torch_dtype(wl.dtype), wl.act)
    print(desc)
    assert "channel_resident" in desc
    full_check(wl)


def test_backward_uses_only_y():
    """The same y bits in a fresh buffer (x long gone) give the same gradients."""
    wl = workloads.config(4).with_shape(4, 16, 10, 10)
    inp = workloads.make_inputs(wl)
    ref = harness.run_gpu(inp)
    y2 = ref.y.clone()
    dy = harness.to_device(inp.dy, wl)
    dx = torch.empty_like(dy)
    C = wl.C
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    si = torch.from_numpy(ref.save_invstd).cuda()
    dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(wl.N, C, wl.H, wl.W, wl.layout, y2.dtype)
    ws.fill_(0xAB)                        # workspace contents on entry do not matter
    iabn.iabn_backward(y2, dy, dx, wl.N, C, wl.H, wl.W, wl.layout, g, b, si, dg, db, wl.act,
                       wl.act_param, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref.dx)
    assert np.array_equal(dg.cpu().numpy(), ref.dgamma)


EVAL = [custom(2, 3, 8, 9, 9), custom(3, 2, 24, 6, 6), custom(4, 3, 8, 5, 5),
        custom(5, 2, 40, 3, 3), custom(2, 3, 7, 5, 3, layout="NHWC", act="elu", act_param=0.7),
        custom(3, 2, 13, 4, 5, dtype="bf16")]


@pytest.mark.parametrize("wl", EVAL, ids=lambda w: w.name)
def test_forward_eval(wl):
    inp = workloads.make_inputs(wl)
    rng = np.random.default_rng(1)
    rm = rng.normal(0, 1, wl.C).astype(np.float32)
    rv = rng.uniform(0.3, 2.0, wl.C).astype(np.float32)
    x = harness.to_device(inp.x, wl)
    iabn.iabn_forward_eval(x, wl.N, wl.C, wl.H, wl.W, wl.layout, torch.from_numpy(inp.gamma).cuda(),
                           torch.from_numpy(inp.beta).cuda(), torch.from_numpy(rm).cuda(),
                           torch.from_numpy(rv).cuda(), wl.act, wl.act_param, wl.eps)
    torch.cuda.synchronize()
    xf = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    o = oracle.forward_eval(xf, inp.gamma, inp.beta, rm, rv, wl.act, harness.f32(wl.act_param),
                            harness.f32(wl.eps), storage=wl.dtype)
    e = harness.rel_err_tensor(harness.to_nchw64(x, wl), o)
    assert e <= harness.TOL[wl.dtype], e


# Backward through the inference forward (frozen running statistics): the GPU's
# own y from iabn_forward_eval, then iabn_backward_eval, against the oracle fed
# those y bits.  With and without dgamma/dbeta; vector and scalar paths; both
# layouts and storage dtypes; dx over dy.
EVAL_BWD = [custom(2, 3, 8, 9, 9), custom(4, 3, 8, 5, 5, act_param=0.7),
            custom(3, 2, 24, 6, 6, layout="NHWC"),
            custom(2, 3, 7, 5, 3, layout="NHWC", act="elu", act_param=0.7),
            custom(3, 2, 13, 4, 5, dtype="bf16", act="identity", act_param=0.0),
            custom(2, 8, 64, 28, 28), custom(3, 4, 256, 16, 16, layout="NHWC"),
            custom(2, 4, 16, 8, 8, dtype="f16", act="elu", act_param=1.0)]


@pytest.mark.parametrize("grads", [True, False], ids=["grads", "dx_only"])
@pytest.mark.parametrize("wl", EVAL_BWD, ids=lambda w: w.name)
def test_backward_eval(wl, grads):
    inp = workloads.make_inputs(wl)
    rng = np.random.default_rng(5)
    rm = rng.normal(0, 1, wl.C).astype(np.float32)
    rv = rng.uniform(0.3, 2.0, wl.C).astype(np.float32)
    N, C, H, W = wl.N, wl.C, wl.H, wl.W
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    rvt = torch.from_numpy(rv).cuda()
    y = harness.to_device(inp.x, wl)
    iabn.iabn_forward_eval(y, N, C, H, W, wl.layout, g, b, torch.from_numpy(rm).cuda(), rvt,
                           wl.act, wl.act_param, wl.eps)
    dy = harness.to_device(inp.dy, wl)
    dx = torch.empty_like(dy)
    dg = torch.empty(C, device="cuda") if grads else None
    db = torch.empty(C, device="cuda") if grads else None
    ws = iabn.workspace(N, C, H, W, wl.layout, y.dtype)
    ws.fill_(0xAB)
    iabn.iabn_backward_eval(y, dy, dx, N, C, H, W, wl.layout, g, b, rvt, wl.eps, dg, db, wl.act,
                            wl.act_param, ws)
    # in place over dy, and the other variant (sums or not), give the same values
    dy2 = harness.to_device(inp.dy, wl)
    dg2 = torch.empty(C, device="cuda") if not grads else None
    db2 = torch.empty(C, device="cuda") if not grads else None
    iabn.iabn_backward_eval(y, dy2, dy2, N, C, H, W, wl.layout, g, b, rvt, wl.eps, dg2, db2,
                            wl.act, wl.act_param, ws)
    torch.cuda.synchronize()
    assert torch.equal(dy2, dx)
    y64 = harness.to_nchw64(y, wl)
    dy64 = workloads.from_storage(inp.dy, N, C, H, W, wl.layout, wl.dtype)
    o = oracle.backward_eval(y64, dy64, inp.gamma, inp.beta, rv, wl.act,
                             harness.f32(wl.act_param), harness.f32(wl.eps))
    errs = {"dx": harness.rel_err_tensor(harness.to_nchw64(dx, wl), o["dx"])}
    if grads:
        errs["dgamma"] = harness.rel_err_vec(dg.cpu().numpy(), o["dgamma"])
        errs["dbeta"] = harness.rel_err_vec(db.cpu().numpy(), o["dbeta"])
    print("case:", wl.name, grads, errs, flush=True)
    harness.assert_within(errs, wl.dtype, "backward_eval " + wl.name)


@pytest.mark.parametrize("W", [64, 63], ids=["vec", "scalar"])
def test_f16_storage_rounds_to_nearest_even(W):
    """fp16 results are rounded to nearest, ties to even, with subnormals and
    overflow to infinity.  With eps = 0, running stats (0, 1), beta = 0 and the
    identity activation, the inference forward is y = x*gamma, exact in fp32 for
    these values, so the one rounding is the storage one and the bits must equal
    the oracle's binary16 rounding of the exact product."""
    base = np.array([1.0, 1.0 + 2 ** -10, 1.0 + 3 * 2 ** -10, 2.0 - 2 ** -10, 2 ** -14,
                     3 * 2 ** -24, 2 ** -24, 1023 * 2 ** -24, 65504.0, -65504.0, 2048.0,
                     0.5 + 2 ** -11, -(1.0 + 2 ** -10), 60000.0, 0.0, -3 * 2 ** -24])
    vals = np.resize(base, W)
    gamma = np.array([1.0 + 2 ** -11, 1.0 - 2 ** -12], np.float32)
    x64 = np.stack([vals, vals])[None, :, None, :]              # N=1, C=2, H=1, W
    wl = custom(2, 1, 2, 1, W, dtype="f16", act="identity", act_param=0.0)
    xs = workloads.to_storage(x64, "NCHW", "f16")
    assert np.array_equal(workloads.from_storage(xs, 1, 2, 1, W, "NCHW", "f16"), x64)
    x = harness.to_device(xs, wl)
    z2 = torch.zeros(2, device="cuda")
    iabn.iabn_forward_eval(x, 1, 2, 1, W, "NCHW", torch.from_numpy(gamma).cuda(), z2, z2,
                           torch.ones(2, device="cuda"), "identity", 0.0, 0.0)
    torch.cuda.synchronize()
    got = harness.to_nchw64(x, wl)
    want = oracle.round_storage(x64 * gamma.astype(np.float64)[None, :, None, None], "f16")
    assert np.array_equal(got, want), (got[0, :, 0, :16], want[0, :, 0, :16])


def test_running_stats_are_optional():
    wl = custom(2, 4, 8, 6, 6)
    inp = workloads.make_inputs(wl)
    x = harness.to_device(inp.x, wl)
    C = wl.C
    sm, si = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(wl.N, C, wl.H, wl.W, wl.layout, x.dtype)
    iabn.iabn_forward_train(x, wl.N, C, wl.H, wl.W, wl.layout,
                            torch.from_numpy(inp.gamma).cuda(), torch.from_numpy(inp.beta).cuda(),
                            None, None, sm, si, wl.act, wl.act_param, wl.eps, wl.momentum, ws)
    torch.cuda.synchronize()
    ref = harness.run_gpu(inp, backward=False)
    assert torch.equal(x, ref.y)
    assert np.array_equal(si.cpu().numpy(), ref.save_invstd)


def test_errors_raise_in_python():
    wl = custom(2, 2, 4, 4, 4)
    x = torch.zeros(harness.storage_shape(wl), device="cuda")
    C = wl.C
    v = torch.ones(C, device="cuda")
    with pytest.raises(iabn.IABNError):
        iabn.iabn_forward_train(x, wl.N, C, wl.H, wl.W, "NCHW", v, v, None, None, v.clone(),
                                v.clone(), "leaky_relu", 0.01, 1e-5, 0.1, None)


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_elu_near_zero_keeps_relative_accuracy(layout):
    """ELU on channels whose pre-activations all sit near 0 (below it): y is then
    tiny, and exp(z) - 1 formed directly would lose most of its digits.  Running
    statistics that match a channel's own, with a small gamma and beta, put z
    in [-1e-3, 1e-3] for the inference forward; the training forward gets the
    same from a small gamma.  Both must stay within the fp32 gate."""
    wl = custom(4, 2, 32, 9, 12, layout=layout, act="elu", act_param=1.0)
    inp = workloads.make_inputs(wl)
    xf = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    rm = xf.mean(axis=(0, 2, 3)).astype(np.float32)
    rv = xf.var(axis=(0, 2, 3)).astype(np.float32)
    gamma = (np.where(np.arange(wl.C) % 2, 1.0, -1.0) * 2e-4).astype(np.float32)
    beta = np.full(wl.C, -1e-4, np.float32)
    x = harness.to_device(inp.x, wl)
    iabn.iabn_forward_eval(x, wl.N, wl.C, wl.H, wl.W, wl.layout, torch.from_numpy(gamma).cuda(),
                           torch.from_numpy(beta).cuda(), torch.from_numpy(rm).cuda(),
                           torch.from_numpy(rv).cuda(), wl.act, wl.act_param, wl.eps)
    torch.cuda.synchronize()
    o = oracle.forward_eval(xf, gamma, beta, rm, rv, wl.act, harness.f32(wl.act_param),
                            harness.f32(wl.eps), storage=wl.dtype)
    assert np.abs(o).max() < 2e-3
    e = harness.rel_err_tensor(harness.to_nchw64(x, wl), o)
    print("eval:", e, flush=True)
    assert e <= harness.TOL[wl.dtype], e
    # training: the same small affine step on the batch's own statistics
    inp.gamma[:] = gamma
    inp.beta[:] = beta
    run = harness.run_gpu(inp)
    ef = harness.check_forward(inp, run)
    ef.update(harness.check_backward(inp, run))
    print("train:", ef, flush=True)
    harness.assert_within(ef, wl.dtype, "train")


@pytest.mark.parametrize("layout,act,W", [("NCHW", "leaky_relu", 8), ("NCHW", "elu", 7),
                                          ("NHWC", "elu", 8), ("NHWC", "identity", 5)])
def test_forward_eval_with_cancelling_terms(layout, act, W):
    """Inference with running statistics far from the batch: running_mean lies
    3000 of the channel's standard deviations below its mean and beta cancels
    the shift, so (x - running_mean)*s and beta are about 3000 times the output.
    Formed plainly in fp32 their rounding alone would put the error near 2e-4 of
    the output; the gate is the fp32 one.  Vector (W = 8) and single-element
    (W odd) paths."""
    wl = custom(2, 3, 24, 6, W, layout=layout, act=act, act_param=1.0 if act == "elu" else 0.01)
    inp = workloads.make_inputs(wl)
    xf = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    mu, sd = xf.mean(axis=(0, 2, 3)), xf.std(axis=(0, 2, 3))
    rm = (mu - 3000.0 * sd).astype(np.float32)
    rv = np.random.default_rng(3).uniform(0.5, 2.0, wl.C).astype(np.float32)
    gamma = np.random.default_rng(4).uniform(0.5, 1.5, wl.C).astype(np.float32)
    s = gamma.astype(np.float64) / np.sqrt(rv.astype(np.float64) + harness.f32(wl.eps))
    beta = (-s * (mu - rm.astype(np.float64))).astype(np.float32)
    x = harness.to_device(inp.x, wl)
    iabn.iabn_forward_eval(x, wl.N, wl.C, wl.H, wl.W, wl.layout, torch.from_numpy(gamma).cuda(),
                           torch.from_numpy(beta).cuda(), torch.from_numpy(rm).cuda(),
                           torch.from_numpy(rv).cuda(), wl.act, wl.act_param, wl.eps)
    torch.cuda.synchronize()
    o = oracle.forward_eval(xf, gamma, beta, rm, rv, wl.act, harness.f32(wl.act_param),
                            harness.f32(wl.eps), storage=wl.dtype)
    assert np.abs(beta).min() > 1000 * np.sqrt(np.mean(o * o))
    e = harness.rel_err_tensor(harness.to_nchw64(x, wl), o)
    print("eval with cancelling terms:", e, flush=True)
    assert e <= harness.TOL[wl.dtype], e


def _ulps(got: np.ndarray, exact: np.ndarray) -> np.ndarray:
    """|got - exact| in units of the fp32 spacing at |exact|."""
    return np.abs(got.astype(np.float64) - exact) / np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)


def test_elu_transcendentals_in_ulps_on_fp32():
    """The fp32 kernels' exp(z) - 1 and log(1 + u), element by element against
    fp64, where the affine step is exact (gamma 1, beta 0, running mean 0 and
    variance 1 with eps 0, so z is the input itself):
    - iabn_forward_eval: y = expm1(x) for x from -87 to -1e-30, within 4 ulp;
    - iabn_backward_eval with one element per channel and dy = 1: dgamma_c =
      (y + 1)*log1p(y) for y from -1 + 2^-24 to -1e-30, within 8 ulp (the
      slope y + 1 and the product add a rounding each)."""
    rng = np.random.default_rng(21)
    z = np.concatenate([-np.logspace(-30, np.log10(87.0), 40000), rng.uniform(-1, 0, 20000),
                        -rng.uniform(0, 1e-3, 5536)]).astype(np.float32)
    n = z.size
    one, zero = torch.ones(1, device="cuda"), torch.zeros(1, device="cuda")
    x = torch.from_numpy(z.copy()).cuda()
    iabn.iabn_forward_eval(x, 1, 1, 1, n, "NCHW", one, zero, zero, one, "elu", 1.0, 0.0)
    torch.cuda.synchronize()
    e = _ulps(x.cpu().numpy(), np.expm1(z.astype(np.float64)))
    print("expm1: max %.2f ulp" % e.max(), flush=True)
    assert e.max() <= 4.0, (e.max(), z[np.argmax(e)])

    y = np.concatenate([-np.logspace(-30, np.log10(1 - 2 ** -24), 40000),
                        rng.uniform(-1, 0, 20000), -rng.uniform(0, 1e-3, 5536)]).astype(np.float32)
    C = y.size
    ones, zeros = torch.ones(C, device="cuda"), torch.zeros(C, device="cuda")
    yt = torch.from_numpy(y.copy()).cuda()
    dy = torch.ones(C, device="cuda")
    dx = torch.empty_like(dy)
    dg, db = torch.empty(C, device="cuda"), torch.empty(C, device="cuda")
    ws = iabn.workspace(1, C, 1, 1, "NCHW", torch.float32)
    iabn.iabn_backward_eval(yt, dy, dx, 1, C, 1, 1, "NCHW", ones, zeros, ones, 0.0, dg, db, "elu",
                            1.0, ws)
    torch.cuda.synchronize()
    y64 = y.astype(np.float64)
    e = _ulps(dg.cpu().numpy(), (y64 + 1.0) * np.log1p(y64))
    print("log1p: max %.2f ulp" % e.max(), flush=True)
    assert e.max() <= 8.0, (e.max(), y[np.argmax(e)])

"""The C-ABI library loads, exports every entry point include/iabn.h declares, and
rejects bad arguments before any HIP call (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iabn.h")

iabn = pytest.importorskip("place_batchnorm_activation_amd")
lib = iabn.lib

OK, INVALID, UNSUPPORTED, WS, MISALIGNED = 0, 1, 2, 3, 4
A = 0x10000  # a 64 KiB-aligned fake device address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(iabn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "iabn_forward_train" in names and "iabn_backward" in names
    assert "iabn_forward_eval" in names and "iabn_workspace_size" in names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert iabn.status_string(0) == "ok"
    assert "workspace" in iabn.status_string(3)
    assert iabn.iabn_version() >= 100


def test_workspace_size_depends_only_on_shape():
    a = lib.iabn_workspace_size(32, 256, 56, 56, 0, 0)
    assert a > 256 * 16
    assert a == lib.iabn_workspace_size(32, 256, 56, 56, 0, 0)
    assert lib.iabn_workspace_size(0, 256, 56, 56, 0, 0) == 0
    assert lib.iabn_workspace_size(2, 0, 4, 4, 0, 0) == 0
    assert lib.iabn_workspace_size(-1, 4, 4, 4, 0, 0) == 0
    assert lib.iabn_workspace_size(2, 4, 4, 4, 7, 0) == 0
    assert lib.iabn_workspace_size(2, 4, 4, 4, 0, 3) == 0          # no dtype 3
    # fp16 and bf16 storage share every size (16-bit elements)
    assert lib.iabn_workspace_size(2, 256, 512, 512, 1, 2) == \
        lib.iabn_workspace_size(2, 256, 512, 512, 1, 1)
    # a plan whose slices are shared by groups of workgroups holds its exchange past
    # the split kernels' sections: 8 bytes per epoch (one per slice, padded to 32)
    # and 4 tagged words per member and channel (64x2048x7x7: 32 slices of eight
    # lanes in groups of 8)
    split = lib.iabn_workspace_size(64, 2048, 7, 7, 1, 1) - 8 * (32 + 4 * 8 * 2048)
    assert split > 0 and split % 256 == 0
    assert lib.iabn_workspace_size(64, 2048, 7, 7, 1, 2) == lib.iabn_workspace_size(64, 2048, 7, 7, 1, 1)
    # partial workspace stays small next to the data (a few percent)
    for (N, C, H, W, lay, dt) in [(32, 256, 56, 56, 0, 0), (2, 256, 512, 512, 1, 1),
                                  (16, 512, 28, 28, 0, 0), (64, 2048, 7, 7, 1, 1)]:
        data = N * C * H * W * (4 if dt == 0 else 2)
        assert lib.iabn_workspace_size(N, C, H, W, lay, dt) < 0.08 * data


def _fwd(x=A, N=2, C=3, H=4, W=4, layout=0, dtype=0, g=A, b=A, rm=A, rv=A, sm=A, si=A,
         act=1, p=0.01, eps=1e-5, mom=0.1, ws=A, wsb=1 << 20):
    return lib.iabn_forward_train(x, N, C, H, W, layout, dtype, g, b, rm, rv, sm, si, act, p, eps,
                                  mom, ws, wsb, None)


def test_forward_train_validation():
    assert _fwd(layout=2) == INVALID
    assert _fwd(dtype=5) == INVALID
    assert _fwd(N=-1) == INVALID
    assert _fwd(act=9) == INVALID
    assert _fwd(p=0.0) == INVALID
    assert _fwd(p=-0.1) == INVALID
    assert _fwd(p=float("nan")) == INVALID
    assert _fwd(act=2, p=-1.0) == INVALID
    assert _fwd(eps=-1e-5) == INVALID
    assert _fwd(eps=float("inf")) == INVALID
    assert _fwd(mom=1.5) == INVALID
    assert _fwd(mom=-0.1) == INVALID
    assert _fwd(rm=None) == INVALID             # running stats: both or neither
    assert _fwd(N=1, H=1, W=1) == INVALID       # m = 1: unbiased variance undefined
    assert _fwd(x=None) == INVALID
    assert _fwd(g=None) == INVALID
    assert _fwd(sm=None) == INVALID
    assert _fwd(x=A + 2) == MISALIGNED          # fp32 element pointer not 4-byte aligned
    assert _fwd(g=A + 1) == MISALIGNED
    assert _fwd(ws=None) == WS
    assert _fwd(wsb=16) == WS
    # a grouped slice-resident plan needs its exchange words: the split kernels'
    # size alone is refused, before any device call
    full = lib.iabn_workspace_size(64, 2048, 7, 7, 1, 1)
    shape = dict(N=64, C=2048, H=7, W=7, layout=1, dtype=1)
    assert _fwd(wsb=full - 8, **shape) == WS
    assert _bwd(wsb=full - 8, dy=A + (1 << 26), dx=A + (1 << 27), **shape) == WS
    assert _fwd(ws=A + 4) == MISALIGNED
    # C == 0 is a no-op that succeeds without touching anything
    assert _fwd(C=0, x=None, g=None, b=None, sm=None, si=None, ws=None) == OK


def test_stage_entry_validation():
    assert lib.iabn_forward_stats(A, 2, 3, 4, 4, 0, 0, A, A, None, None, A, A, -1.0, 0.1, A,
                                  1 << 20, None) == INVALID
    assert lib.iabn_forward_apply(A, 2, 3, 4, 4, 0, 0, 1, 0.0, A, 1 << 20, None) == INVALID
    assert lib.iabn_forward_apply(A, 2, 3, 4, 4, 0, 0, 1, 0.01, None, 0, None) == WS
    assert lib.iabn_backward_reduce(A, A, 2, 3, 4, 4, 0, 0, A, A, None, A, A, 1, 0.01, A,
                                    1 << 20, None) == INVALID
    assert lib.iabn_backward_apply(A, A, A + 64, 2, 3, 4, 4, 0, 0, 1, 0.01, None, 0, None) == INVALID


def test_forward_eval_validation():
    ev = lib.iabn_forward_eval
    assert ev(A, 2, 3, 4, 4, 0, 0, A, A, A, None, 1, 0.01, 1e-5, None) == INVALID
    assert ev(A, 2, 3, 4, 4, 0, 1, A, A, A, A, 1, 0.01, -1.0, None) == INVALID
    assert ev(A + 1, 2, 3, 4, 4, 0, 1, A, A, A, A, 1, 0.01, 1e-5, None) == MISALIGNED
    # empty tensors are a no-op
    assert ev(None, 0, 3, 4, 4, 0, 0, None, None, None, None, 1, 0.01, 1e-5, None) == OK
    assert ev(None, 2, 3, 0, 4, 1, 1, None, None, None, None, 2, 1.0, 1e-5, None) == OK


def _bwd(y=A, dy=2 * A, dx=3 * A, N=2, C=3, H=4, W=4, layout=0, dtype=0, g=A, b=A, si=A, dg=A,
         db=A, act=1, p=0.01, ws=A, wsb=1 << 20):
    return lib.iabn_backward(y, dy, dx, N, C, H, W, layout, dtype, g, b, si, dg, db, act, p, ws,
                             wsb, None)


def test_backward_validation():
    assert _bwd(dtype=3) == INVALID
    assert _bwd(dtype=2, y=A + 1) == MISALIGNED
    assert _bwd(act=1, p=0.0) == INVALID
    assert _bwd(dx=A) == INVALID                 # dx aliases y
    assert _bwd(dx=A + 64) == INVALID            # dx overlaps y
    assert _bwd(dx=2 * A + 64) == INVALID        # dx partly overlaps dy
    assert _bwd(N=1, H=1, W=1) == INVALID
    assert _bwd(g=None) == INVALID
    assert _bwd(si=None) == INVALID
    assert _bwd(ws=None) == WS
    assert _bwd(dtype=1, y=A + 1) == MISALIGNED
    assert _bwd(C=0, y=None, dy=None, dx=None, g=None, b=None, si=None, dg=None, db=None,
                ws=None) == OK


def _bev(y=A, dy=2 * A, dx=3 * A, N=2, C=3, H=4, W=4, layout=0, dtype=0, g=A, b=A, rv=A,
         eps=1e-5, dg=A, db=A, act=1, p=0.01, ws=A, wsb=1 << 20):
    return lib.iabn_backward_eval(y, dy, dx, N, C, H, W, layout, dtype, g, b, rv, eps, dg, db,
                                  act, p, ws, wsb, None)


def test_backward_eval_validation():
    assert _bev(act=2, p=-1.0) == INVALID
    assert _bev(eps=-1e-3) == INVALID
    assert _bev(eps=float("nan")) == INVALID
    assert _bev(dg=None) == INVALID             # dgamma and dbeta: both or neither
    assert _bev(rv=None) == INVALID
    assert _bev(dx=A) == INVALID                # dx aliases y
    assert _bev(dx=2 * A + 64) == INVALID       # dx partly overlaps dy
    assert _bev(N=0) == INVALID                 # m = 0 with channels
    assert _bev(ws=None) == WS
    assert _bev(dtype=1, dy=2 * A + 1) == MISALIGNED
    assert _bev(C=0, y=None, dy=None, dx=None, g=None, b=None, rv=None, dg=None, db=None,
                ws=None) == OK


def test_plan_choice_for_the_workloads():
    """Which kernels each workload runs (host-side plan; no GPU needed)."""
    d = iabn.iabn_describe_plan
    assert d(32, 256, 56, 56, "NCHW", iabn.F32, "leaky_relu") == \
        "forward=channel_resident(512x49) backward=channel_resident(512x49,dy_streamed)"
    assert d(32, 256, 56, 56, "NCHW", iabn.F32, "leaky_relu") == \
        d(32, 256, 56, 56, "NCHW", iabn.F32, "identity")
    assert d(16, 512, 28, 28, "NCHW", iabn.F32, "elu").startswith(
        "forward=channel_resident(256x13) backward=channel_resident(256x13,dy_resident)")
    assert d(2, 4, 8, 8, "NCHW", iabn.F32, "leaky_relu").startswith("forward=channel_resident")
    # a map too large to hold: 256 workgroups in groups of 64, eight lanes per row,
    # keep part of it in registers and stream the rest
    assert d(2, 256, 512, 512, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_streamed(512x8x(28+16)+4,group64) " \
        "backward=split(reduce:256x256,apply:256x256,vec16)"
    # ... the backward too while half its rows stay resident
    assert d(32, 256, 56, 56, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_streamed(512x8x(28+16)+4,group64) backward=slice_streamed(512x8x(14+8)+2,group64)"
    assert d(4, 2048, 56, 56, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_streamed(512x8x(28+16)+4,group8) backward=slice_streamed(512x8x(14+8)+2,group8)"
    # four lanes per row where 16-byte vectors make 16 per pixel
    assert d(1, 128, 360, 360, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_streamed(512x4x(28+16)+4,group64) backward=slice_streamed(512x4x(14+8)+2,group64)"
    # ... but not two lanes per row: split, the backward sums on one workgroup per CU
    assert d(32, 64, 112, 112, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=split(stats:256x256,apply:512x256,vec16) " \
        "backward=split(reduce:256x256,apply:512x256,vec16)"
    # eight lanes per row (whole lines) in groups of 8
    assert d(64, 2048, 7, 7, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_resident(512x8x7,group8) backward=slice_resident(512x8x7,group8)"
    # ... but four lanes where eight would leave 4 rows a thread
    assert d(32, 2048, 7, 7, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_resident(512x4x4,group4) backward=slice_resident(512x4x4,group4)"
    # too many rows for a workgroup to hold: split
    assert d(2, 16, 80, 80, "NHWC", iabn.F32, "leaky_relu").startswith("forward=split")
    # few slices on a large tensor: split
    assert d(16, 16, 28, 28, "NHWC", iabn.BF16, "leaky_relu").startswith("forward=split")
    # fp16 storage plans exactly as bf16
    for shape in ((64, 2048, 7, 7, "NHWC"), (2, 256, 512, 512, "NHWC"), (16, 512, 28, 28, "NCHW"),
                  (32, 256, 56, 56, "NCHW")):
        assert d(*shape, torch.float16, "leaky_relu") == d(*shape, torch.bfloat16, "leaky_relu")
    # planes off the vector width (7x7) keep channels resident element by element
    assert d(32, 2048, 7, 7, "NCHW", iabn.F32, "leaky_relu") == \
        "forward=channel_resident_scalar(256x8) backward=channel_resident_scalar(256x8,dy_resident)"
    assert d(3, 5, 17, 19, "NCHW", iabn.F32, "leaky_relu").startswith(
        "forward=channel_resident_scalar(256x4)")
    # ... and so do misaligned pointers, up to 24576 elements per channel; beyond
    # that the scalar split path
    assert d(32, 512, 7, 7, "NCHW", iabn.F32, "leaky_relu", aligned16=False).startswith(
        "forward=channel_resident_scalar")
    assert "split" in d(32, 256, 56, 56, "NCHW", iabn.F32, "leaky_relu", aligned16=False)
    assert "scalar)" in d(32, 256, 56, 56, "NCHW", iabn.F32, "leaky_relu", aligned16=False)
    # NHWC maps with more rows than a workgroup holds share each slice among a
    # group of workgroups (within the 256 CUs)
    assert d(32, 1024, 14, 14, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_resident(512x4x7,group8) backward=slice_resident(512x4x7,group8)"
    assert d(32, 512, 28, 28, "NHWC", iabn.BF16, "leaky_relu").startswith(
        "forward=slice_resident(512x4x13,group16)")
    assert d(32, 512, 7, 7, "NHWC", iabn.BF16, "leaky_relu").startswith("forward=slice_resident")
    # tensors under 4 MB: one lane per row, as many workgroups as the CUs take
    assert d(8, 2048, 7, 7, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_resident(256x1x2) backward=slice_resident(256x1x2)"
    assert d(32, 256, 14, 14, "NHWC", iabn.BF16, "leaky_relu") == \
        "forward=slice_resident(256x1x4,group8) backward=slice_resident(256x1x4,group8)"
    # 8 slices of two lanes, groups of 32
    assert d(32, 128, 56, 56, "NHWC", iabn.BF16, "leaky_relu").startswith("forward=slice_")
    # ELU takes the same channel-resident variants
    assert "channel_resident(512x49)" in d(32, 256, 56, 56, "NCHW", iabn.F32, "elu")
    with pytest.raises(ValueError):
        d(2, 4, 4, 4, "NCHW", iabn.F32, 9)


def test_grouped_kernels_can_be_switched_off():
    """With the grouped kernels forbidden, no plan has workgroups that wait on one
    another, and the workspace size does not change (host-side plan only)."""
    d = iabn.iabn_describe_plan
    shapes = [(64, 2048, 7, 7, "NHWC", iabn.BF16), (2, 256, 512, 512, "NHWC", iabn.BF16),
              (32, 1024, 14, 14, "NHWC", iabn.BF16), (32, 256, 56, 56, "NHWC", iabn.BF16),
              (32, 64, 112, 112, "NCHW", iabn.F32), (16, 512, 28, 28, "NCHW", iabn.F32),
              (32, 256, 56, 56, "NCHW", iabn.F32)]
    sizes = [lib.iabn_workspace_size(N, C, H, W, 0 if lay == "NCHW" else 1, dt)
             for (N, C, H, W, lay, dt) in shapes]
    before = iabn.iabn_set_grouped_kernels(None)
    try:
        assert iabn.iabn_set_grouped_kernels(True) == before
        assert "group" in d(64, 2048, 7, 7, "NHWC", iabn.BF16, "leaky_relu")
        assert "group" in d(32, 64, 112, 112, "NCHW", iabn.F32, "leaky_relu")
        assert iabn.iabn_set_grouped_kernels(False) is True
        assert iabn.iabn_set_grouped_kernels(None) is False
        for (N, C, H, W, lay, dt) in shapes:
            plan = d(N, C, H, W, lay, dt, "leaky_relu")
            assert "group" not in plan and "slice_streamed" not in plan, plan
        # the tail map keeps its slices on chip, one workgroup per slice
        assert d(64, 2048, 7, 7, "NHWC", iabn.BF16, "leaky_relu") == \
            "forward=slice_resident(512x2x13) backward=slice_resident(512x2x13)"
        assert d(2, 256, 512, 512, "NHWC", iabn.BF16, "leaky_relu").startswith("forward=split")
        # channels a workgroup holds stay resident without groups
        assert d(32, 256, 56, 56, "NCHW", iabn.F32, "leaky_relu") == \
            "forward=channel_resident(512x49) backward=channel_resident(512x49,dy_streamed)"
        for (N, C, H, W, lay, dt), n in zip(shapes, sizes):
            assert lib.iabn_workspace_size(N, C, H, W, 0 if lay == "NCHW" else 1, dt) == n
    finally:
        iabn.iabn_set_grouped_kernels(before)
    assert iabn.iabn_set_grouped_kernels(None) == before


def test_workspace_status_validation():
    flag = ctypes.c_int(7)
    assert lib.iabn_workspace_status(A, 1 << 20, 0, None, None) == INVALID
    assert lib.iabn_workspace_status(None, 1 << 20, 0, ctypes.byref(flag), None) == WS
    assert flag.value == 0
    assert lib.iabn_workspace_status(A, 255, 0, ctypes.byref(flag), None) == WS
    assert lib.iabn_workspace_status(A + 8, 1 << 20, 0, ctypes.byref(flag), None) == MISALIGNED


def test_noalloc_forward_rejects_shapes_beyond_its_scratch():
    """The no-allocation forward rejects, before any HIP call, a shape whose
    workspace exceeds its static scratch, and validates like iabn_forward_train."""
    big = (1, 1 << 20, 16, 16)                    # NHWC bf16: 24 MiB of workspace
    assert lib.iabn_workspace_size(*big, 1, 1) > iabn.NOALLOC_SCRATCH_BYTES
    assert lib.iabn_forward_train_noalloc(A, *big, 1, 1, A, A, A, A, A, A, 1, 0.01, 1e-5, 0.1,
                                          None) == WS
    assert lib.iabn_workspace_size(64, 2048, 7, 7, 1, 1) <= iabn.NOALLOC_SCRATCH_BYTES
    assert lib.iabn_workspace_size(2, 256, 512, 512, 1, 1) <= iabn.NOALLOC_SCRATCH_BYTES
    # argument errors as for iabn_forward_train, before any HIP call
    assert lib.iabn_forward_train_noalloc(A, 2, 3, 4, 4, 0, 0, A, A, A, A, A, A, 1, 0.0, 1e-5,
                                          0.1, None) == INVALID
    assert lib.iabn_forward_train_noalloc(A, 2, 3, 4, 4, 0, 0, None, A, A, A, A, A, 1, 0.01, 1e-5,
                                          0.1, None) == INVALID
    assert lib.iabn_forward_train_noalloc(A, 1, 3, 1, 1, 0, 0, A, A, A, A, A, A, 1, 0.01, 1e-5,
                                          0.1, None) == INVALID           # m = 1
    assert lib.iabn_forward_train_noalloc(A + 2, 2, 3, 4, 4, 0, 0, A, A, A, A, A, A, 1, 0.01,
                                          1e-5, 0.1, None) == MISALIGNED
    assert lib.iabn_forward_train_noalloc(None, 2, 0, 4, 4, 0, 0, None, None, None, None, None,
                                          None, 1, 0.01, 1e-5, 0.1, None) == OK


def test_ckpt_validation():
    """Optimized checkpointing entry points validate like their InPlace-ABN
    counterparts, plus y must not overlap x."""
    def fwd(x=A, y=8 * A, N=2, C=3, H=4, W=4, ws=A, wsb=1 << 20, p=0.01):
        return lib.iabn_forward_train_ckpt(x, y, N, C, H, W, 0, 0, A, A, A, A, A, A, 1, p, 1e-5,
                                           0.1, ws, wsb, None)
    assert fwd(y=None) == INVALID
    assert fwd(y=A + 64) == INVALID                 # y overlaps x
    assert fwd(p=0.0) == INVALID
    assert fwd(N=1, H=1, W=1) == INVALID            # m = 1
    assert fwd(ws=None) == WS
    assert fwd(y=8 * A + 2) == MISALIGNED
    assert fwd(C=0, x=None, y=None) == OK

    def rec(xh=A, y=8 * A, C=3, p=0.01):
        return lib.iabn_recompute_from_xhat(xh, y, 2, C, 4, 4, 0, 0, A, A, 1, p, None)
    assert rec(y=None) == INVALID
    assert rec(y=A + 64) == INVALID                 # partly overlaps xhat
    assert rec(p=-1.0) == INVALID
    assert rec(C=0, xh=None, y=None) == OK

    def bwd(xh=A, dy=4 * A, dx=8 * A, ws=A):
        return lib.iabn_backward_ckpt(xh, dy, dx, 2, 3, 4, 4, 0, 0, A, A, A, A, A, 1, 0.01, ws,
                                      1 << 20, None)
    assert bwd(dx=A) == INVALID                     # dx over xhat
    assert bwd(dx=4 * A + 64) == INVALID            # dx partly over dy
    assert bwd(ws=None) == WS


def test_module_rejects_parameters_it_cannot_read():
    """The autograd module hands weight, bias and the running statistics to the
    library as float32 pointers: other dtypes or sizes are refused before any call."""
    import torch
    from place_batchnorm_activation_amd.autograd import InPlaceABN
    x = torch.randn(2, 8, 4, 4)
    m = InPlaceABN(8).half()
    with pytest.raises(TypeError, match="float32"):
        m(x.half())
    m = InPlaceABN(8)
    m.running_var = torch.ones(8, dtype=torch.float64)
    with pytest.raises(TypeError, match="float32"):
        m(x)
    m = InPlaceABN(6)
    with pytest.raises(TypeError, match="of 8 elements.*got torch.float32 \\(6,\\)"):
        m(x)


@pytest.mark.parametrize("value,grouped", [("0", False), ("1", True), (None, True)])
def test_grouped_kernels_environment_switch(value, grouped):
    """IABN_GROUPED_KERNELS=0, read when a fresh process first plans a call, forbids
    the kernels whose workgroups wait on one another (any other value, or none,
    allows them)."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("IABN_GROUPED_KERNELS", None)
    if value is not None:
        env["IABN_GROUPED_KERNELS"] = value
    code = ("import sys; sys.path.insert(0, %r); import torch; "
            "import place_batchnorm_activation_amd as i; "
            "print(i.iabn_describe_plan(64, 2048, 7, 7, 'NHWC', torch.bfloat16, 'leaky_relu')); "
            "print(i.iabn_set_grouped_kernels(None))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    plan, setting = out.stdout.split("\n")[:2]
    assert ("group" in plan) == grouped, plan
    assert setting == str(grouped)


def test_module_geometry_of_any_batchnorm_input():
    """How the autograd module presents [N, C, *] tensors to the library (host
    only): spatial extents fold into H*W; channels_last(_3d) tensors are NHWC."""
    import torch
    from place_batchnorm_activation_amd.autograd import _geometry
    assert _geometry(torch.empty(8, 16)) == (8, 16, 1, 1, "NCHW")
    assert _geometry(torch.empty(4, 16, 10)) == (4, 16, 10, 1, "NCHW")
    assert _geometry(torch.empty(2, 3, 4, 5)) == (2, 3, 4, 5, "NCHW")
    assert _geometry(torch.empty(2, 3, 4, 5, 6)) == (2, 3, 120, 1, "NCHW")
    cl = torch.empty(2, 3, 4, 5).contiguous(memory_format=torch.channels_last)
    assert _geometry(cl) == (2, 3, 4, 5, "NHWC")
    cl3 = torch.empty(2, 3, 4, 5, 6).contiguous(memory_format=torch.channels_last_3d)
    assert _geometry(cl3) == (2, 3, 20, 6, "NHWC")
    # one channel: both memory formats coincide, and NCHW is taken
    assert _geometry(torch.empty(2, 1, 4, 5).contiguous(memory_format=torch.channels_last))[4] == \
        "NCHW"
    with pytest.raises(ValueError):
        _geometry(torch.empty(8))
    with pytest.raises(ValueError):
        _geometry(torch.empty(4, 10, 16).transpose(1, 2))


def test_module_state_dict_matches_batchnorm2d():
    """The module's state dict has BatchNorm2d's keys for every option, so
    checkpoints load either way (host only)."""
    import torch
    from place_batchnorm_activation_amd.autograd import InPlaceABN
    for affine in (True, False):
        for track in (True, False):
            a = InPlaceABN(8, affine=affine, track_running_stats=track)
            b = torch.nn.BatchNorm2d(8, affine=affine, track_running_stats=track)
            assert sorted(a.state_dict()) == sorted(b.state_dict()), (affine, track)
    a = InPlaceABN(8)
    b = torch.nn.BatchNorm2d(8)
    b.num_batches_tracked.fill_(7)
    b.running_var.fill_(2.0)
    a.load_state_dict(b.state_dict())
    assert a._steps == 7 and float(a.running_var[0]) == 2.0


def test_binding_refuses_per_channel_vectors_of_other_dtypes():
    """The library reads gamma, beta, statistics and gradients as float32: the
    binding refuses a float64 (or any other) vector instead of passing its bytes
    on (host only; the refusal comes before any library call)."""
    import torch
    x = torch.empty(2 * 3 * 4 * 4)
    v32 = torch.empty(3)
    v64 = torch.empty(3, dtype=torch.float64)
    ws = torch.empty(1 << 16, dtype=torch.uint8)
    with pytest.raises(TypeError, match="float32"):
        iabn.iabn_forward_train(x, 2, 3, 4, 4, "NCHW", v64, v32, None, None, v32, v32,
                                "leaky_relu", 0.01, 1e-5, 0.1, ws, stream=0)
    with pytest.raises(TypeError, match="float32"):
        iabn.iabn_backward(x, x, x, 2, 3, 4, 4, "NCHW", v32, v32, v32, v32,
                           v32.half(), "leaky_relu", 0.01, ws, stream=0)

"""The planner and the workspace size over many seeded random shapes (CPU only).

Without a device every compute entry point stops at its first HIP call, which
fails (IABN_ERR_HIP); everything before it -- validation, planning and the
workspace check -- runs as on a GPU.  So a call that reaches the launch was
given a large enough workspace: iabn_workspace_size must satisfy every entry
point that takes one, for every activation and with the exchanging kernels on
or off (the size does not depend on that setting).  The pointers are fake,
non-overlapping, aligned addresses that nothing dereferences."""
import random

import pytest

iabn = pytest.importorskip("place_batchnorm_activation_amd")
lib = iabn.lib

HIP_ERR = 5
ACTS = ((0, 0.0), (1, 0.01), (2, 1.0))


def _shapes(n, seed):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        N = rng.choice([1, 2, 3, 4, 8, 16, 32, 64])
        C = rng.choice([1, 2, 3, 4, 7, 8, 16, 24, 32, 64, 96, 128, 256, 512, 1024, 2048])
        H = rng.choice([1, 2, 3, 5, 7, 8, 14, 17, 28, 56, 64, 112, 150, 224])
        W = rng.choice([H, H, rng.randint(1, 230)])
        if N * H * W < 2 or N * C * H * W > (1 << 27):
            continue
        out.append((N, C, H, W, rng.randint(0, 1), rng.randint(0, 2)))
    return out


def _calls(N, C, H, W, layout, dtype, act, a, ws):
    """(name, status) of every entry point that takes a workspace, on fake
    buffers: x/y at X, dy at DY, dx at DX, y of the checkpointing forward at Y2,
    per-channel vectors at V + k * vb, the workspace at WS."""
    esize = 4 if dtype == 0 else 2
    tb = (N * C * H * W * esize + 4095) & ~4095
    X = 1 << 36
    DY, DX, Y2 = X + tb, X + 2 * tb, X + 3 * tb
    V = X + 4 * tb
    vb = (C * 4 + 255) & ~255
    g, b, rm, rv, sm, si, dg, db = (V + k * vb for k in range(8))
    WS = V + 8 * vb
    shape = (N, C, H, W, layout, dtype)
    return [
        ("forward_train", lib.iabn_forward_train(X, *shape, g, b, rm, rv, sm, si, act, a, 1e-5,
                                                 0.1, WS, ws, None)),
        ("forward_stats", lib.iabn_forward_stats(X, *shape, g, b, rm, rv, sm, si, 1e-5, 0.1, WS,
                                                 ws, None)),
        ("forward_apply", lib.iabn_forward_apply(X, *shape, act, a, WS, ws, None)),
        ("backward", lib.iabn_backward(X, DY, DX, *shape, g, b, si, dg, db, act, a, WS, ws,
                                       None)),
        ("backward_in_place", lib.iabn_backward(X, DY, DY, *shape, g, b, si, dg, db, act, a, WS,
                                                ws, None)),
        ("backward_reduce", lib.iabn_backward_reduce(X, DY, *shape, g, b, si, dg, db, act, a, WS,
                                                     ws, None)),
        ("backward_apply", lib.iabn_backward_apply(X, DY, DX, *shape, act, a, WS, ws, None)),
        ("backward_eval", lib.iabn_backward_eval(X, DY, DX, *shape, g, b, rv, 1e-5, dg, db, act,
                                                 a, WS, ws, None)),
        ("forward_train_ckpt", lib.iabn_forward_train_ckpt(X, Y2, *shape, g, b, rm, rv, sm, si,
                                                           act, a, 1e-5, 0.1, WS, ws, None)),
        ("backward_ckpt", lib.iabn_backward_ckpt(X, DY, DX, *shape, g, b, si, dg, db, act, a, WS,
                                                 ws, None)),
    ]


@pytest.mark.parametrize("grouped", [True, False])
def test_workspace_size_suffices_for_every_entry_point(grouped):
    before = iabn.iabn_set_grouped_kernels(grouped)
    try:
        for (N, C, H, W, layout, dtype) in _shapes(250, 11 if grouped else 12):
            ws = lib.iabn_workspace_size(N, C, H, W, layout, dtype)
            assert ws >= 256, (N, C, H, W, layout, dtype)
            for act, a in ACTS:
                for name, st in _calls(N, C, H, W, layout, dtype, act, a, ws):
                    assert st == HIP_ERR, (name, N, C, H, W, layout, dtype, act,
                                           iabn.status_string(st))
                buf_ok = iabn.iabn_describe_plan(N, C, H, W, layout, dtype, act)
                assert buf_ok.startswith("forward=") and " backward=" in buf_ok
    finally:
        iabn.iabn_set_grouped_kernels(before)


def test_noalloc_forward_takes_exactly_the_shapes_its_scratch_holds():
    """iabn_forward_train_noalloc reaches the launch when the shape's workspace fits
    the static scratch and refuses it (IABN_ERR_WORKSPACE) otherwise, before any
    device call."""
    X = 1 << 36
    seen = {True: 0, False: 0}
    rng = random.Random(14)
    wide = [(rng.choice([1, 2, 4]), rng.choice([1 << 16, 3 << 16, 1 << 18, 1 << 20]),
             rng.choice([2, 4, 8, 16]), rng.choice([2, 4, 8, 16]), rng.randint(0, 1),
             rng.randint(0, 2)) for _ in range(120)]
    for (N, C, H, W, layout, dtype) in _shapes(300, 13) + wide:
        need = lib.iabn_workspace_size(N, C, H, W, layout, dtype)
        fits = need <= iabn.NOALLOC_SCRATCH_BYTES
        V = X + ((N * C * H * W * 4 + 4095) & ~4095)
        vb = (C * 4 + 255) & ~255
        st = lib.iabn_forward_train_noalloc(X, N, C, H, W, layout, dtype, V, V + vb, None, None,
                                            V + 2 * vb, V + 3 * vb, 1, 0.01, 1e-5, 0.1, None)
        assert st == (HIP_ERR if fits else 3), (N, C, H, W, layout, dtype, need)
        seen[fits] += 1
    assert seen[True] > 100 and seen[False] > 20, seen

"""The library called from C++ alone (tests/c_caller.cpp, built by build() into
tests/_bin/): no Python and no PyTorch in the calling process, which sizes and
allocates its own workspace and runs on a HIP stream of its own.  Its outputs
must be the bits the Python binding gets for the same problem on the same
device, and within the oracle's gates (the forward on the same x bits, the
backward on the program's own y bits)."""
import dataclasses
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import harness
import workloads

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "_bin", "c_caller")
LAYOUT = {"NCHW": 0, "NHWC": 1}
DTYPE = {"f32": 0, "bf16": 1, "f16": 2}
ACT = {"identity": 0, "leaky_relu": 1, "elu": 2}

CASES = [
    workloads.config(1),                                             # tiny NCHW fp32
    workloads.config(4).with_shape(4, 16, 20, 20),                   # NCHW fp32 ELU
    dataclasses.replace(workloads.config(2).with_shape(2, 8, 12, 12), dtype="f16"),
    workloads.config(3).with_shape(3, 64, 24, 24),                   # NHWC bf16
    workloads.config(5).with_shape(16, 512, 7, 7),                   # NHWC bf16, grouped
]


def _problem(inp) -> bytes:
    wl = inp.wl
    head = b"IABNCALL" + struct.pack("<4q3i3f", wl.N, wl.C, wl.H, wl.W, LAYOUT[wl.layout],
                                     DTYPE[wl.dtype], ACT[wl.act], wl.act_param, wl.eps,
                                     wl.momentum)
    vecs = [np.ascontiguousarray(v, dtype=np.float32).tobytes()
            for v in (inp.gamma, inp.beta, inp.running_mean, inp.running_var)]
    return head + inp.x.tobytes() + inp.dy.tobytes() + b"".join(vecs)


def _outputs(raw: bytes, wl):
    nb = wl.numel * wl.esize
    assert len(raw) == 2 * nb + 6 * 4 * wl.C + 4, len(raw)
    dt = workloads.storage_torch_dtype(wl.dtype)
    shape = harness.storage_shape(wl)

    def tensor(off):
        return torch.frombuffer(bytearray(raw[off:off + nb]), dtype=dt).reshape(shape)

    vec = np.frombuffer(raw, dtype=np.float32, count=6 * wl.C, offset=2 * nb).reshape(6, wl.C)
    timed_out = struct.unpack("<i", raw[-4:])[0]
    return tensor(0), tensor(nb), vec, timed_out


@pytest.mark.parametrize("wl", CASES, ids=lambda w: "%s_%dx%dx%dx%d_%s" % (
    w.name, w.N, w.C, w.H, w.W, w.dtype))
def test_c_caller_matches_the_binding_and_the_oracle(wl, tmp_path):
    assert os.path.exists(BIN), "tests/_bin/c_caller is built by __graft_entry__.build()"
    inp = workloads.make_inputs(wl)
    problem, outputs = tmp_path / "problem.bin", tmp_path / "outputs.bin"
    problem.write_bytes(_problem(inp))
    print("case:", wl.name, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype, wl.act, flush=True)
    r = subprocess.run([BIN, str(problem), str(outputs)], capture_output=True, text=True,
                       timeout=60)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    y, dx, vec, timed_out = _outputs(outputs.read_bytes(), wl)
    assert timed_out == 0
    sm, si, rm, rv, dg, db = vec

    # the same calls through the Python binding, in this process
    ref = harness.run_gpu(inp)
    assert torch.equal(y, ref.y.cpu())
    assert torch.equal(dx, ref.dx.cpu())
    for got, want in ((sm, ref.save_mean), (si, ref.save_invstd), (rm, ref.running_mean),
                      (rv, ref.running_var), (dg, ref.dgamma), (db, ref.dbeta)):
        assert np.array_equal(got, want)

    # and the oracle's gates on the program's own outputs
    run = harness.GpuRun(y=y, dx=dx, save_mean=sm.copy(), save_invstd=si.copy(),
                         running_mean=rm.copy(), running_var=rv.copy(), dgamma=dg.copy(),
                         dbeta=db.copy())
    errs = harness.check_forward(inp, run)
    errs.update(harness.check_backward(inp, run))
    print("  ", errs, flush=True)
    harness.assert_within(errs, wl.dtype, wl.name)

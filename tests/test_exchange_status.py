"""The exchange status word and the switch that forbids grouped kernels, on the
GPU through the C ABI: a recorded timeout is reported and cleared; with grouped
kernels switched off the ungrouped plans run and match the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import harness
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import place_batchnorm_activation_amd as iabn

TIMEOUT_WORD = 0x69616E6254494D45          # the value a timed-out wait stores


def test_status_word_reports_and_clears():
    ws = iabn.workspace(64, 2048, 7, 7, "NHWC", torch.bfloat16)
    ws.zero_()
    assert iabn.iabn_workspace_status(ws) is False
    ws[:8].view(torch.int64).fill_(TIMEOUT_WORD)
    assert iabn.iabn_workspace_status(ws, clear=False) is True
    assert iabn.iabn_workspace_status(ws, clear=True) is True      # read, then cleared
    assert iabn.iabn_workspace_status(ws) is False
    ws[:8].view(torch.int64).fill_(TIMEOUT_WORD)
    with pytest.raises(iabn.ExchangeTimeout):
        iabn.check_workspace(ws)
    iabn.check_workspace(ws)                                        # cleared by the check
    # a grouped call on a workspace of garbage: no timeout, word left clear
    ws.random_(0, 256)
    ws[:8].zero_()
    wl = workloads.config(5)
    inp = workloads.make_inputs(wl)
    run = harness.run_gpu(inp, ws=ws)                               # asserts the word clear
    harness.assert_within(harness.check_forward(inp, run), "bf16", "forward")


UNGROUPED = [workloads.config(5), workloads.config(3),
             dataclasses.replace(workloads.config(2).with_shape(8, 64, 112, 112),
                                 name="resnet_stage1_nchw_f32_8x64x112x112"),
             dataclasses.replace(workloads.config(3).with_shape(32, 1024, 14, 14),
                                 name="resnet_stage4_nhwc_bf16_32x1024x14x14")]


@pytest.mark.parametrize("wl", UNGROUPED, ids=lambda w: w.name)
def test_ungrouped_plans_match_the_oracle(wl):
    dt = workloads.storage_torch_dtype(wl.dtype)
    grouped = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout, dt, wl.act)
    before = iabn.iabn_set_grouped_kernels(False)
    try:
        plan = iabn.iabn_describe_plan(wl.N, wl.C, wl.H, wl.W, wl.layout, dt, wl.act)
        print("case:", wl.name, "grouped:", grouped, "switched off:", plan, flush=True)
        assert "group" not in plan and "slice_streamed" not in plan
        inp = workloads.make_inputs(wl)
        run = harness.run_gpu(inp)
    finally:
        iabn.iabn_set_grouped_kernels(before)
    block = 32 if wl.storage_bytes > (128 << 20) else wl.C
    errs = harness.check_all_channels(inp, run, block)
    print("  ", errs, flush=True)
    harness.assert_within(errs, wl.dtype, wl.name)
    # the grouped plan again, on the same input: equal within the tolerance
    run2 = harness.run_gpu(inp)
    tol = harness.TOL[wl.dtype]
    for c0 in range(0, wl.C, block):
        sel = slice(c0, min(wl.C, c0 + block))
        assert harness.rel_err_tensor(harness.to_nchw64(run2.y, wl, sel),
                                      harness.to_nchw64(run.y, wl, sel)) <= tol
        assert harness.rel_err_tensor(harness.to_nchw64(run2.dx, wl, sel),
                                      harness.to_nchw64(run.dx, wl, sel)) <= tol
    assert np.all(np.isfinite(run.save_invstd)) and np.all(np.isfinite(run2.save_invstd))

"""The five workloads of the selective-scan study at full size, through the C
ABI, against the fp64 oracle: completely where the oracle finishes in
seconds, else on sampled channels (every time step of each sampled channel)."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import TOL, assert_close, gather_channels, log, run_gpu, sample_channels

pytestmark = pytest.mark.gpu


def run_workload(name, nsample):
    w = synth.WORKLOADS[name]
    log("workload %s" % name)
    inp = synth.workload_inputs(name, seed=0)
    y, h, g = run_gpu(inp, bidir=w["bidir"], want_h=True, want_g=w["bidir"])
    tol = TOL[w["dtype"]]
    if nsample is None:
        y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=w["bidir"], want_h_last=True, want_g_first=w["bidir"])
        assert_close("y", y, y_ref, tol)
        assert_close("h_last", h, h_ref, TOL["f32"])
        if w["bidir"]:
            assert_close("g_first", g, g_ref, TOL["f32"])
        return
    chans = sample_channels(w["Bs"], w["ED"], nsample)
    y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=w["bidir"], chans=chans, want_h_last=True,
                                      want_g_first=w["bidir"])
    assert_close("y[sampled channels]", gather_channels(y, chans, w["ED"]), y_ref, tol)
    Bi, Ei = np.divmod(chans, w["ED"])
    assert_close("h_last[sampled]", h[Bi, Ei], h_ref, TOL["f32"])
    if w["bidir"]:
        assert_close("g_first[sampled]", g[Bi, Ei], g_ref, TOL["f32"])


def test_page_shape():
    run_workload("fwd_f32_Bs2_L64_ED64_N16", None)


def test_fp32_8x1024x1536_with_final_state():
    run_workload("fwd_f32_Bs8_L1024_ED1536_N16", None)


def test_bf16_4x8192x5120():
    run_workload("fwd_bf16_Bs4_L8192_ED5120_N16", 256)


def test_fp32_long_sequence_131072():
    run_workload("fwd_f32_Bs1_L131072_ED2048_N16", 64)


def test_bidirectional_8x4096x1536():
    run_workload("bidir_f32_Bs8_L4096_ED1536_N16", 256)


def test_bidirectional_long_sequence_131072():
    run_workload("bidir_f32_Bs1_L131072_ED2048_N16", 64)


def run_bwd_workload(name):
    from parity_util import assert_grads_close, run_gpu_bwd
    w = synth.WORKLOADS[name]
    log("backward workload %s" % name)
    inp = synth.workload_inputs(name, seed=0)
    dy = synth.make_output_grad(w["Bs"], w["L"], w["ED"], w["dtype"], seed=0)
    got = run_gpu_bwd(inp, dy, want_dh0=True, bidir=w["bidir"])
    ref = oracle.scan_bwd(**inp, dy=dy, bidir=w["bidir"])
    assert_grads_close(got, ref, w["dtype"])


def test_backward_fp32_8x1024x1536():
    run_bwd_workload("bwd_f32_Bs8_L1024_ED1536_N16")


def test_backward_bf16_4x8192x5120():
    run_bwd_workload("bwd_bf16_Bs4_L8192_ED5120_N16")


def test_backward_long_sequence_131072():
    run_bwd_workload("bwd_f32_Bs1_L131072_ED2048_N16")


def test_backward_bidirectional_8x4096x1536():
    run_bwd_workload("bwd_bidir_f32_Bs8_L4096_ED1536_N16")


def run_train_workload(name):
    """The training step: the forward scan keeps the round states, the
    backward reads them; every gradient against the oracle's adjoint."""
    from parity_util import assert_grads_close, run_gpu_bwd
    w = synth.WORKLOADS[name]
    log("training-step workload %s" % name)
    inp = synth.workload_inputs(name, seed=0)
    dy = synth.make_output_grad(w["Bs"], w["L"], w["ED"], w["dtype"], seed=0)
    got = run_gpu_bwd(inp, dy, want_dh0=True, use_ckpt=True, bidir=w["bidir"])
    ref = oracle.scan_bwd(**inp, dy=dy, bidir=w["bidir"])
    assert_grads_close(got, ref, w["dtype"])


def test_training_step_fp32_8x1024x1536():
    run_train_workload("train_f32_Bs8_L1024_ED1536_N16")


def test_training_step_bf16_4x8192x5120():
    run_train_workload("train_bf16_Bs4_L8192_ED5120_N16")


def test_training_step_long_sequence_131072():
    run_train_workload("train_f32_Bs1_L131072_ED2048_N16")


def test_training_step_bidirectional_8x4096x1536():
    run_train_workload("train_bidir_f32_Bs8_L4096_ED1536_N16")

"""GPU parity of the carried states in both directions: the reverse
direction's initial state g0 of the bidirectional scans, and the gradients
of the final states (dh_last; dg_first and dg0 for the bidirectional
backward), the per-direction final_states and dfinal_states of "Some
questions of Bi-Mamba2 and Hydra" (the MambaChunkScanCombinedFn listings).
Each against the oracle on the same seeded inputs, and sequences cut in two
pieces, forward and backward, against the whole."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import (TOL, assert_close, assert_grads_close, log, options_inputs, run_gpu, run_gpu_bwd,
                         run_gpu_ssd)

pytestmark = pytest.mark.gpu


def states(seed, stream, shape, scale=1.0):
    return (scale * synth.normal(seed, stream, shape)).astype(np.float32)


def piece(inp, lo, hi):
    return {k: (np.ascontiguousarray(v[:, lo:hi]) if v.ndim == 3 else v) for k, v in inp.items()}


# --- forward: g0 -------------------------------------------------------------
@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 64, 64, "f32"), (2, 301, 40, "f32"), (3, 257, 96, "bf16"),
                                           (1, 1, 16, "f32")])
def test_bidirectional_reverse_initial_state(Bs, L, ED, dtype):
    log("case bidir g0 %dx%dx%d %s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L + ED)
    h0, g0 = states(L, 80, (Bs, ED, 16)), states(L, 81, (Bs, ED, 16))
    y, h, g = run_gpu(inp, bidir=True, want_h=True, want_g=True, h0=h0, g0=g0)
    y_ref, h_ref, g_ref = oracle.scan(**inp, h0=h0, g0=g0, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])


def test_bidirectional_reverse_initial_state_with_options():
    inp, opts = options_inputs(2, 200, 48, "f32", seed=61)
    g0 = states(61, 82, (2, 48, 16))
    y, _, g = run_gpu(inp, bidir=True, want_g=True, g0=g0, opts=opts)
    y_ref, _, g_ref = oracle.scan(**inp, g0=g0, bidir=True, want_g_first=True, **opts)
    assert_close("y", y, y_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidirectional_sequence_in_two_pieces(dtype):
    # the reverse state flows from the later piece into the earlier one and
    # the forward state the other way: a call on the later piece gives its
    # g_first (independent of its h0), the earlier piece runs from it and
    # gives h_last, the later piece runs again from that
    Bs, L, ED, L1 = 2, 700, 64, 333
    log("case bidir two pieces %s" % dtype)
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=62)
    p1, p2 = piece(inp, 0, L1), piece(inp, L1, L)
    _, _, g2 = run_gpu(p2, bidir=True, want_g=True)
    y1, h1, g1 = run_gpu(p1, bidir=True, want_h=True, want_g=True, g0=g2)
    y2, h2, _ = run_gpu(p2, bidir=True, want_h=True, h0=h1)
    y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y", np.concatenate([y1, y2], axis=1), y_ref, TOL[dtype])
    assert_close("h_last", h2, h_ref, TOL["f32"])
    assert_close("g_first", g1, g_ref, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multihead_bidirectional_reverse_initial_state(dtype):
    Bs, L, H, P, G, N = 2, 100, 4, 64, 2, 64
    log("case multi-head bidir g0 %s" % dtype)
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, dtype, seed=63)
    h0, g0 = states(63, 83, (Bs, H, P, N), 0.3), states(63, 84, (Bs, H, P, N), 0.3)
    y, h, g = run_gpu_ssd(inp, h0=h0, g0=g0, want_h=True, bidir=True, want_g=True)
    y_ref, h_ref, g_ref = oracle.ssd(**inp, h0=h0, g0=g0, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])


# --- backward: dh_last, dg_first, dg0 -----------------------------------------
@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 64, 64, "f32"), (2, 301, 40, "f32"), (2, 257, 96, "bf16"),
                                           (1, 1, 16, "f32")])
def test_final_state_gradient(Bs, L, ED, dtype):
    log("case bwd dh_last %dx%dx%d %s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L + 3)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=L + 3)
    h0, dhl = states(L, 85, (Bs, ED, 16)), states(L, 86, (Bs, ED, 16))
    got = run_gpu_bwd(inp, dy, h0=h0, want_dh0=True, dh_last=dhl)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h0, dh_last=dhl)
    assert_grads_close(got, ref, dtype)


def test_final_state_gradient_only():
    # dy = 0: every gradient comes from the final state alone
    Bs, L, ED = 2, 150, 64
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=64)
    dy = np.zeros((Bs, L, ED), np.float32)
    dhl = states(64, 87, (Bs, ED, 16))
    got = run_gpu_bwd(inp, dy, want_dh0=True, dh_last=dhl)
    ref = oracle.scan_bwd(**inp, dy=dy, dh_last=dhl)
    assert_grads_close(got, ref, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_of_a_sequence_in_two_pieces(dtype):
    # training a sequence cut in two: the later piece's dh0 enters the earlier
    # piece as its dh_last; the pieces' gradients make up the whole's
    Bs, L, ED, L1 = 2, 640, 64, 257
    log("case bwd two pieces %s" % dtype)
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=65)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=65)
    p1, p2 = piece(inp, 0, L1), piece(inp, L1, L)
    _, h1, _ = run_gpu(p1, want_h=True)
    g2 = run_gpu_bwd(p2, np.ascontiguousarray(dy[:, L1:]), h0=h1, want_dh0=True)
    g1 = run_gpu_bwd(p1, np.ascontiguousarray(dy[:, :L1]), want_dh0=True, dh_last=g2["dh0"])
    ref = oracle.scan_bwd(**inp, dy=dy)
    whole = {k: np.concatenate([g1[k], g2[k]], axis=1) for k in ("dx", "ddelta", "dB", "dC")}
    whole["dA"] = g1["dA"] + g2["dA"]
    whole["dD"] = g1["dD"] + g2["dD"]
    whole["dh0"] = g1["dh0"]
    assert_grads_close(whole, ref, dtype)


@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 64, 64, "f32"), (2, 301, 40, "f32"), (2, 257, 96, "bf16")])
def test_bidirectional_state_gradients(Bs, L, ED, dtype):
    log("case bidir bwd states %dx%dx%d %s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L + 5)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=L + 5)
    sh = (Bs, ED, 16)
    h0, g0, dhl, dgf = states(L, 88, sh), states(L, 89, sh), states(L, 90, sh), states(L, 91, sh)
    got = run_gpu_bwd(inp, dy, h0=h0, want_dh0=True, bidir=True, g0=g0, dh_last=dhl, dg_first=dgf, want_dg0=True)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h0, g0=g0, dh_last=dhl, dg_first=dgf, bidir=True)
    assert_grads_close(got, ref, dtype)


def test_bidirectional_state_gradients_with_options_and_gate():
    inp, opts = options_inputs(2, 200, 48, "f32", seed=66)
    dy = synth.make_output_grad(2, 200, 48, "f32", seed=66)
    sh = (2, 48, 16)
    g0, dhl, dgf = states(66, 92, sh), states(66, 93, sh), states(66, 94, sh)
    got = run_gpu_bwd(inp, dy, want_dh0=True, bidir=True, g0=g0, dh_last=dhl, dg_first=dgf, want_dg0=True, **opts)
    ref = oracle.scan_bwd(**inp, dy=dy, g0=g0, dh_last=dhl, dg_first=dgf, bidir=True, **opts)
    assert_grads_close(got, ref, "f32")


@pytest.mark.parametrize("Bs,L,ED", [(2, 0, 48), (0, 17, 48)])
def test_empty_sequence_carries_the_states(Bs, L, ED):
    # over zero steps: g_first = g0, dh0 = dh_last, dg0 = dg_first
    log("case empty states %dx%dx%d" % (Bs, L, ED))
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=67)
    sh = (Bs, ED, 16)
    g0, dhl, dgf = states(67, 95, sh), states(67, 96, sh), states(67, 97, sh)
    _, _, g = run_gpu(inp, bidir=True, want_g=True, g0=g0)
    assert_close("g_first", g, g0.astype(np.float64), 0.0)
    dy = synth.make_output_grad(Bs, L, ED, "f32", seed=67)
    got = run_gpu_bwd(inp, dy, want_dh0=True, bidir=True, g0=g0, dh_last=dhl, dg_first=dgf, want_dg0=True)
    ref = oracle.scan_bwd(**inp, dy=dy, g0=g0, dh_last=dhl, dg_first=dgf, bidir=True)
    assert_grads_close(got, ref, "f32")
    np.testing.assert_array_equal(got["dh0"], dhl.astype(np.float64))
    np.testing.assert_array_equal(got["dg0"], dgf.astype(np.float64))

"""GPU parity of the backward passes (ssm_scan_bwd, ssm_scan_bidir_bwd)
against the oracle's adjoint (oracle.scan_bwd, bidir=False / True) on the
same seeded inputs."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import assert_grads_close, degenerate_inputs, log, options_inputs, run_gpu_bwd

pytestmark = pytest.mark.gpu


def check(Bs, L, ED, dtype="f32", seed=0, h0=False, D_none=False, want_dD=True, bidir=False):
    log("bwd case Bs=%d L=%d ED=%d dtype=%s seed=%d h0=%s D_none=%s bidir=%s" % (Bs, L, ED, dtype, seed, h0, D_none,
                                                                               bidir))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=seed)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=seed)
    h = synth.normal(seed, 79, (Bs, ED, 16)) if h0 else None
    got = run_gpu_bwd(inp, dy, h0=h, D_none=D_none, want_dD=want_dD, want_dh0=True, bidir=bidir)
    ref_inp = dict(inp, D=None) if D_none else inp
    ref = oracle.scan_bwd(**ref_inp, dy=dy, h0=h, bidir=bidir)
    assert_grads_close(got, ref, dtype)
    return got


def test_page_shape():
    check(2, 64, 64)


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 64, 65, 200, 1009])
def test_sequence_lengths(L):
    check(2, L, 64, seed=L)


@pytest.mark.parametrize("ED", [16, 20, 48, 100, 130])
def test_channel_counts(ED):
    check(2, 77, ED, seed=ED)


def test_bf16():
    check(2, 300, 96, dtype="bf16", seed=5)


@pytest.mark.parametrize("case", ["no_decay", "full_decay", "growth", "zero_steps", "zero_input", "mixed"])
def test_degenerate_inputs(case):
    log("bwd degenerate case %s" % case)
    inp = degenerate_inputs(case, L=150, ED=48)
    dy = synth.make_output_grad(2, 150, 48, "f32", seed=14)
    got = run_gpu_bwd(inp, dy, want_dD=True, want_dh0=True)
    ref = oracle.scan_bwd(**inp, dy=dy)
    assert_grads_close(got, ref, "f32")


def test_initial_state():
    check(2, 150, 64, seed=6, h0=True)


def test_no_D():
    check(2, 70, 32, seed=7, D_none=True)


def test_no_dD():
    check(2, 70, 32, seed=8, want_dD=False)


def test_many_batch_rows():
    check(9, 40, 48, seed=9)


def test_repeatable_bits():
    inp = synth.make_inputs(3, 257, 80, 16, "f32", seed=10)
    dy = synth.make_output_grad(3, 257, 80, "f32", seed=10)
    a = run_gpu_bwd(inp, dy, want_dh0=True)
    b = run_gpu_bwd(inp, dy, want_dh0=True)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_training_shape_full():
    # the forward training shape (Bs 8, L 1024, ED 1536, N 16), every gradient compared in full
    check(8, 1024, 1536, seed=11, h0=True)


@pytest.mark.parametrize("Bs,L,ED", [(2, 0, 48), (0, 17, 48), (2, 17, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_of_empty_inputs(Bs, L, ED, dtype):
    """An empty output has zero gradients everywhere (dA, dD, dh0; dB and dC
    when there are steps but no channels), as the oracle gives."""
    log("backward empty case Bs=%d L=%d ED=%d dtype=%s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=42)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=42)
    h0 = synth.normal(42, 9, (Bs, ED, 16))
    got = run_gpu_bwd(inp, dy, h0=h0, want_dh0=True)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h0)
    assert_grads_close(got, ref, dtype)


# ---- bidirectional backward -------------------------------------------------
def test_bidir_page_shape():
    check(2, 64, 64, bidir=True)


@pytest.mark.parametrize("L", [1, 2, 31, 33, 200, 1009])
def test_bidir_sequence_lengths(L):
    check(2, L, 64, seed=L + 100, bidir=True)


@pytest.mark.parametrize("ED", [20, 130])
def test_bidir_channel_counts(ED):
    check(2, 77, ED, seed=ED + 100, bidir=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidir_initial_state_and_no_D(dtype):
    check(2, 150, 64, dtype=dtype, seed=106, h0=True, bidir=True)
    check(2, 70, 32, dtype=dtype, seed=107, D_none=True, bidir=True)


def test_bidir_bf16():
    check(2, 300, 96, dtype="bf16", seed=105, bidir=True)


@pytest.mark.parametrize("case", ["no_decay", "full_decay", "growth", "mixed"])
def test_bidir_degenerate_inputs(case):
    log("bidir bwd degenerate case %s" % case)
    inp = degenerate_inputs(case, L=150, ED=48)
    dy = synth.make_output_grad(2, 150, 48, "f32", seed=15)
    got = run_gpu_bwd(inp, dy, want_dD=True, want_dh0=True, bidir=True)
    ref = oracle.scan_bwd(**inp, dy=dy, bidir=True)
    assert_grads_close(got, ref, "f32")


def test_bidir_repeatable_bits():
    inp = synth.make_inputs(3, 257, 80, 16, "bf16", seed=110)
    dy = synth.make_output_grad(3, 257, 80, "bf16", seed=110)
    a = run_gpu_bwd(inp, dy, want_dh0=True, bidir=True)
    b = run_gpu_bwd(inp, dy, want_dh0=True, bidir=True)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_bidir_training_shape_full():
    # the bidirectional training shape of the forward (Bs 8, L 4096, ED 1536)
    # at a quarter of the length, every gradient compared in full
    check(8, 1024, 1536, seed=111, h0=True, bidir=True)


# ---- backward through the step-size options (bias, softplus, clamp) ---------
def keep_clear_of_bounds(inp, opts):
    """The clamp's derivative jumps at its bounds; a step mapped to within
    rounding of one could be taken on different sides by the float32 kernel
    and the fp64 oracle. Steps that land within 1e-5 (relative) of a bound --
    the same mapping written in numpy -- are scaled by 1 - 2^-6 until none
    does; the inputs are otherwise unchanged."""
    bf16 = inp["delta"].dtype == np.uint16
    raw = synth.from_bf16(inp["delta"]) if bf16 else inp["delta"].astype(np.float32)
    for _ in range(8):
        v = raw.astype(np.float64)
        if opts.get("dt_bias") is not None:
            v = v + opts["dt_bias"].astype(np.float32).astype(np.float64)
        if opts.get("dt_softplus"):
            v = np.logaddexp(0.0, v)
        bad = np.zeros(v.shape, dtype=bool)
        for bound in opts.get("dt_limit", ()):
            if np.isfinite(bound):
                bad |= np.abs(v - bound) <= 1e-5 * abs(bound)
        if not bad.any():
            return dict(inp, delta=synth.to_bf16(raw) if bf16 else raw)
        raw = raw.copy()
        raw[bad] *= np.float32(1 - 2.0 ** -6)
        if bf16:
            raw = synth.from_bf16(synth.to_bf16(raw))
    raise AssertionError("steps stay on a clamp bound")


def check_options(Bs, L, ED, dtype, seed, opts, bidir=False, h0=False, inp=None):
    log("bwd options case Bs=%d L=%d ED=%d dtype=%s seed=%d bidir=%s options=%s" % (
        Bs, L, ED, dtype, seed, bidir, sorted(opts)))
    if inp is None:
        inp, _ = options_inputs(Bs, L, ED, dtype, seed)
    inp = keep_clear_of_bounds(inp, opts)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=seed)
    h = synth.normal(seed, 79, (Bs, ED, 16)) if h0 else None
    got = run_gpu_bwd(inp, dy, h0=h, want_dh0=True, bidir=bidir, **opts)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h, bidir=bidir, **opts)
    assert ("ddt_bias" in got) == (opts.get("dt_bias") is not None)
    assert ("dz" in got) == (opts.get("z") is not None)
    assert_grads_close(got, ref, dtype)


@pytest.mark.parametrize("Bs,L,ED,dtype,bidir", [(2, 300, 64, "f32", False), (2, 301, 40, "f32", False),
                                                 (2, 257, 64, "bf16", False), (2, 200, 64, "f32", True),
                                                 (2, 150, 48, "bf16", True), (1, 2100, 32, "f32", False)])
def test_step_size_options(Bs, L, ED, dtype, bidir):
    _, opts = options_inputs(Bs, L, ED, dtype, seed=L + ED)
    opts.pop("z")
    check_options(Bs, L, ED, dtype, L + ED, opts, bidir=bidir, h0=True)


def test_step_size_options_each_alone():
    inp, opts = options_inputs(2, 150, 32, "f32", seed=5)
    positive = synth.make_inputs(2, 150, 32, 16, "f32", seed=5)["delta"]   # log-uniform steps
    singles = {"dt_bias": dict(dt_bias=np.abs(opts["dt_bias"]) * 0.02),
               "dt_softplus": dict(dt_softplus=True),
               "dt_limit": dict(dt_limit=(0.01, 0.05)),
               "dt_min": dict(dt_limit=(0.02, float("inf"))),
               "bias_and_limit": dict(dt_bias=np.abs(opts["dt_bias"]) * 0.02, dt_limit=(0.01, 0.05))}
    for key, one in singles.items():
        # raw steps only through softplus; otherwise positive steps
        inp2 = inp if key == "dt_softplus" else dict(inp, delta=positive)
        check_options(2, 150, 32, "f32", 5, one, inp=inp2)


def test_step_size_options_training_shape():
    # (Bs 8, L 1024, ED 1536) with bias, softplus and clamp
    _, opts = options_inputs(8, 1024, 1536, "bf16", seed=12)
    opts.pop("z")
    check_options(8, 1024, 1536, "bf16", 12, opts)


# ---- backward through the output gate ---------------------------------------
@pytest.mark.parametrize("Bs,L,ED,dtype,bidir", [(2, 300, 64, "f32", False), (2, 257, 40, "bf16", False),
                                                 (2, 200, 64, "f32", True), (2, 150, 48, "bf16", True)])
def test_gate_with_step_size_options(Bs, L, ED, dtype, bidir):
    _, opts = options_inputs(Bs, L, ED, dtype, seed=L + ED + 7)
    check_options(Bs, L, ED, dtype, L + ED + 7, opts, bidir=bidir, h0=True)


@pytest.mark.parametrize("bidir", [False, True])
def test_gate_alone(bidir):
    # positive log-uniform steps, no other option; z ~ N(0, 1) and a few
    # large |z| where the gate saturates (silu(z) ~ z, or ~ 0)
    inp = synth.make_inputs(2, 150, 32, 16, "f32", seed=31)
    z = synth.normal(31, 22, (2, 150, 32))
    z[:, ::17, :] *= 30.0
    check_options(2, 150, 32, "f32", 31, dict(z=z), bidir=bidir, inp=inp)


def test_gate_training_shape():
    # (Bs 8, L 1024, ED 1536), bf16, with every option
    _, opts = options_inputs(8, 1024, 1536, "bf16", seed=13)
    check_options(8, 1024, 1536, "bf16", 13, opts)


# ---- split sweeps: long sequences with few channel groups --------------------
# Such sweeps are cut into chunks: a first kernel forms each chunk's
# aggregates from zero states (the sum of its step sizes, the forward state at
# its end, the adjoint at its start), then every chunk runs the backward of
# its own steps from the states folded in from the chunks on either side.

@pytest.mark.parametrize("Bs,L,ED,dtype,bidir", [(1, 3000, 64, "f32", False), (1, 5000, 42, "f32", False),
                                                 (2, 4096, 32, "bf16", False), (1, 3000, 64, "f32", True),
                                                 (2, 4096, 32, "bf16", True)])
def test_split_sweep(Bs, L, ED, dtype, bidir):
    log("bwd split case Bs=%d L=%d ED=%d dtype=%s bidir=%s" % (Bs, L, ED, dtype, bidir))
    seed = L + ED + (7 if bidir else 0)
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=seed)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=seed)
    h0 = synth.normal(seed, 79, (Bs, ED, 16))
    dhl = synth.normal(seed, 80, (Bs, ED, 16))
    kw = dict(g0=synth.normal(seed, 81, (Bs, ED, 16)), dg_first=synth.normal(seed, 82, (Bs, ED, 16))) \
        if bidir else {}
    got = run_gpu_bwd(inp, dy, h0=h0, want_dh0=True, bidir=bidir, dh_last=dhl, want_dg0=bidir, **kw)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h0, bidir=bidir, dh_last=dhl, **kw)
    assert_grads_close(got, ref, dtype)


@pytest.mark.parametrize("dtype,bidir", [("f32", False), ("bf16", False), ("f32", True)])
def test_split_sweep_with_options_and_gate(dtype, bidir):
    _, opts = options_inputs(1, 4500, 48, dtype, seed=45)
    check_options(1, 4500, 48, dtype, 45, opts, bidir=bidir, h0=True)


@pytest.mark.parametrize("case", ["no_decay_exact", "full_decay", "zero_steps"])
def test_split_sweep_degenerate_inputs(case):
    # Carries over whole chunks: A = 0 with unit steps and inputs in {-1, 0, 1},
    # where every state, adjoint and gradient is an integer that float32 holds
    # exactly, whatever the order of the sums (with real-valued inputs and no
    # decay over thousands of steps, float32 rounding of the growing sums alone
    # exceeds the tolerance on ddelta where it cancels, split or not: the
    # short unsplit cases above cover those inputs); no carries at all (a
    # underflows to 0); zero steps at every other time.
    log("bwd split degenerate case %s" % case)
    L, ED = 2200, 48
    if case == "no_decay_exact":
        inp = synth.make_inputs(1, L, ED, 16, "f32", seed=16)
        tern = lambda stream, shape: np.sign(np.round(synth.normal(16, stream, shape))).astype(np.float32)
        inp.update(x=tern(40, (1, L, ED)), B=tern(41, (1, L, 16)), C=tern(42, (1, L, 16)),
                   delta=np.ones((1, L, ED), np.float32), A=np.zeros((ED, 16), np.float32),
                   D=np.round(inp["D"]).astype(np.float32))
        dy = tern(43, (1, L, ED))
    else:
        inp = degenerate_inputs(case, Bs=1, L=L, ED=ED)
        dy = synth.make_output_grad(1, L, ED, "f32", seed=16)
    got = run_gpu_bwd(inp, dy, want_dD=True, want_dh0=True)
    ref = oracle.scan_bwd(**inp, dy=dy)
    assert_grads_close(got, ref, "f32")

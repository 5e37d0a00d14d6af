"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import (TOL, assert_close, degenerate_inputs, gather_channels, log, options_inputs, run_gpu,
                         sample_channels)

pytestmark = pytest.mark.gpu


def check_full(Bs, L, ED, dtype="f32", bidir=False, seed=0, D_none=False):
    log("case Bs=%d L=%d ED=%d dtype=%s bidir=%s seed=%d" % (Bs, L, ED, dtype, bidir, seed))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=seed)
    y, h, g = run_gpu(inp, bidir=bidir, want_h=True, want_g=bidir, D_none=D_none)
    ref_inp = dict(inp, D=None) if D_none else inp
    y_ref, h_ref, g_ref = oracle.scan(**ref_inp, bidir=bidir, want_h_last=True, want_g_first=bidir)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])
    if bidir:
        assert_close("g_first", g, g_ref, TOL["f32"])


def test_page_shape_forward():
    check_full(2, 64, 64)


def test_page_shape_bidirectional():
    check_full(2, 64, 64, bidir=True)


@pytest.mark.parametrize("L", [1, 2, 3, 63, 64, 65, 127, 1009])
def test_sequence_lengths(L):
    check_full(2, L, 128, seed=L)


@pytest.mark.parametrize("L", [1, 5, 129, 1009])
def test_sequence_lengths_bidirectional(L):
    check_full(1, L, 64, bidir=True, seed=L)


@pytest.mark.parametrize("ED", [16, 48, 64, 80, 192, 1040])
def test_channel_counts(ED):
    check_full(3, 200, ED, seed=ED)


@pytest.mark.parametrize("ED,dtype,bidir", [(1, "f32", False), (3, "f32", False), (37, "f32", False),
                                             (150, "f32", False), (37, "bf16", False), (150, "bf16", False),
                                             (37, "f32", True), (150, "bf16", True)])
def test_channel_counts_not_multiple_of_4(ED, dtype, bidir):
    # element-by-element loads and stores of the channel chunks (no 16-byte vectors)
    check_full(2, 133, ED, dtype=dtype, bidir=bidir, seed=ED + 1)


def test_split_sequence_channels_not_multiple_of_4():
    check_full(1, 3000, 37, seed=11)


@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("case", ["no_decay", "full_decay", "growth", "zero_steps", "zero_input", "mixed"])
def test_degenerate_inputs(case, bidir):
    log("degenerate case %s bidir=%s" % (case, bidir))
    inp = degenerate_inputs(case)
    y, h, g = run_gpu(inp, bidir=bidir, want_h=True, want_g=bidir)
    y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=bidir, want_h_last=True, want_g_first=bidir)
    assert_close("y", y, y_ref, TOL["f32"])
    assert_close("h_last", h, h_ref, TOL["f32"])
    if bidir:
        assert_close("g_first", g, g_ref, TOL["f32"])
    if case == "zero_input":
        assert np.all(y == 0.0) and np.all(h == 0.0)


def test_single_batch_row_long():
    check_full(1, 4099, 256, seed=5)


def test_bf16_forward():
    check_full(2, 300, 256, dtype="bf16", seed=6)


def test_bf16_bidirectional():
    check_full(2, 300, 128, dtype="bf16", bidir=True, seed=7)


def test_without_D():
    check_full(2, 100, 64, D_none=True, seed=8)
    check_full(2, 100, 64, D_none=True, bidir=True, seed=9)


@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 300, 8192, "f32"), (2, 301, 6150, "f32"), (3, 257, 5120, "bf16")])
def test_more_workgroups_than_three_per_cu(Bs, L, ED, dtype):
    # more than 768 (batch row, channel group) pairs: the launch takes the
    # kernel built for four workgroups per compute unit (vectorised and, with
    # ED not a multiple of 4, element-wise staging)
    check_full(Bs, L, ED, dtype=dtype, seed=ED + L)


def test_repeatable_bitwise():
    inp = synth.make_inputs(2, 777, 192, 16, "f32", seed=10)
    y1, h1, _ = run_gpu(inp, want_h=True)
    y2, h2, _ = run_gpu(inp, want_h=True)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_on_a_side_stream():
    import torch
    inp = synth.make_inputs(2, 130, 64, 16, "f32", seed=11)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y, _, _ = run_gpu(inp, stream=s)
    y_ref, _, _ = oracle.scan(**inp)
    assert_close("y", y, y_ref, TOL["f32"])


# ---- sequences split across workgroups (few channels, long L) ----------------
# With fewer than two (batch row, 16-channel group) pairs per compute unit the
# forward scan cuts the sequence into chunks that hand their end states on and
# correct the start of their output. These shapes take that path.

@pytest.mark.parametrize("Bs,L,ED,dtype", [(1, 3000, 64, "f32"), (1, 5000, 40, "f32"), (2, 4096, 32, "bf16"),
                                           (1, 20000, 128, "f32")])
def test_split_sequence(Bs, L, ED, dtype):
    check_full(Bs, L, ED, dtype=dtype, seed=L + ED)


# The bidirectional scan splits such sequences too: every chunk runs both
# directions from its own entering states (zero inside the sequence), then a
# second kernel folds the chunks' aggregates into the states entering each
# chunk from either side and corrects both ends of its output.

@pytest.mark.parametrize("Bs,L,ED,dtype", [(1, 3000, 64, "f32"), (1, 5000, 42, "f32"), (2, 4096, 32, "bf16"),
                                           (1, 20000, 128, "f32")])
def test_bidirectional_split_sequence(Bs, L, ED, dtype):
    import state_space_model_selective_amd as ssm
    split = ssm.ssm_scan_workspace_bytes(Bs, L, ED, 16, ssm.SSM_F32 if dtype == "f32" else ssm.SSM_BF16, bidir=1)
    plain = 0 if dtype == "f32" else -(-Bs * L * ED * 4 // 256) * 256
    assert split > plain, "this shape is expected to split the sequence"
    log("case bidir split Bs=%d L=%d ED=%d %s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L + ED + 1)
    h0 = (0.5 * synth.normal(L, 70, (Bs, ED, 16))).astype(np.float32)
    g0 = (0.5 * synth.normal(L, 71, (Bs, ED, 16))).astype(np.float32)
    for states in (False, True):
        kw = dict(h0=h0, g0=g0) if states else {}
        y, h, g = run_gpu(inp, bidir=True, want_h=True, want_g=True, **kw)
        y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True, **kw)
        assert_close("y", y, y_ref, TOL[dtype])
        assert_close("h_last", h, h_ref, TOL["f32"])
        assert_close("g_first", g, g_ref, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidirectional_split_with_options_and_gate(dtype):
    log("case bidir split, options %s" % dtype)
    inp, opts = options_inputs(1, 4500, 48, dtype, seed=44)
    y, h, g = run_gpu(inp, bidir=True, want_h=True, want_g=True, opts=opts)
    y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True, **opts)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])


def test_bidirectional_split_slow_decay_and_negative_steps():
    # corrections that run over whole chunks from both ends (tiny steps, A = 0
    # for some states), and mixed-sign step sizes (no early stop)
    log("case bidir split, slow decay / mixed sign")
    inp = synth.make_inputs(1, 6000, 64, 16, "f32", seed=23)
    inp["delta"] = (inp["delta"] * 1e-3).astype(np.float32)
    inp["A"][:, :3] = 0.0
    y, h, g = run_gpu(inp, bidir=True, want_h=True, want_g=True)
    y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y", y, y_ref, TOL["f32"])
    assert_close("h_last", h, h_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])
    inp = synth.make_inputs(1, 4000, 64, 16, "f32", seed=24)
    sign = np.where(synth.uniform(24, 9, inp["delta"].shape, 0, 1) < 0.1, -1.0, 1.0).astype(np.float32)
    inp["delta"] = (inp["delta"] * sign).astype(np.float32)
    y, h, g = run_gpu(inp, bidir=True, want_h=True, want_g=True)
    y_ref, h_ref, g_ref = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y", y, y_ref, TOL["f32"])
    assert_close("h_last", h, h_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])


def test_split_sequence_slow_decay_and_no_decay():
    # tiny step sizes (the carried state decays over the whole chunk) and
    # A = 0 for some states (no decay at all): the correction runs to the end
    log("case split, slow decay")
    inp = synth.make_inputs(1, 6000, 64, 16, "f32", seed=21)
    inp["delta"] = (inp["delta"] * 1e-3).astype(np.float32)
    inp["A"][:, :3] = 0.0
    y, h, _ = run_gpu(inp, want_h=True)
    y_ref, h_ref, _ = oracle.scan(**inp, want_h_last=True)
    assert_close("y", y, y_ref, TOL["f32"])
    assert_close("h_last", h, h_ref, TOL["f32"])


def test_split_sequence_negative_steps():
    # raw step sizes may be negative (the pages pass randn): the early stop of
    # the correction must not trigger then
    log("case split, mixed-sign delta")
    inp = synth.make_inputs(1, 4000, 64, 16, "f32", seed=22)
    sign = np.where(synth.uniform(22, 9, inp["delta"].shape, 0, 1) < 0.1, -1.0, 1.0).astype(np.float32)
    inp["delta"] = (inp["delta"] * sign).astype(np.float32)
    y, h, _ = run_gpu(inp, want_h=True)
    y_ref, h_ref, _ = oracle.scan(**inp, want_h_last=True)
    assert_close("y", y, y_ref, TOL["f32"])
    assert_close("h_last", h, h_ref, TOL["f32"])


def test_split_sequence_status_and_forced_give_up(monkeypatch):
    # The status query reports a clean hand-off for a normal call. Then the
    # hand-off wait's spin limit is forced to zero from the host
    # (SSM_SPLIT_SPIN_LIMIT), so a wait gives up unless its predecessor has
    # already published: every give-up must show as SSM_ERR_HANDOFF and as
    # NaN outputs, and a call without one must still match the oracle. The
    # kernel itself never hangs or faults either way.
    import torch
    import state_space_model_selective_amd as ssm
    from parity_util import to_device, y_to_numpy
    Bs, L, ED, N = 1, 20000, 128, 16
    need = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, ssm.SSM_F32)
    assert need > 0, "this shape is expected to split the sequence"
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=23)
    y_ref, h_ref, _ = oracle.scan(**inp, want_h_last=True)
    dev = torch.device("cuda:0")
    t = to_device(inp, dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for spin in (None, "0", "0", "0"):
        if spin is None:
            monkeypatch.delenv("SSM_SPLIT_SPIN_LIMIT", raising=False)
        else:
            monkeypatch.setenv("SSM_SPLIT_SPIN_LIMIT", spin)
        log("case split status, spin limit %s" % spin)
        h = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)
        y = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], h_last=h, workspace=ws)
        rc = ssm.ssm_scan_fwd_status(t["x"], t["A"], ws)
        yn, hn = y_to_numpy(y), h.double().cpu().numpy()
        log("  status %d, NaN in y: %s" % (rc, bool(np.isnan(yn).any())))
        if spin is None:
            assert rc == ssm.SSM_OK
        if rc == ssm.SSM_OK:
            assert_close("y", yn, y_ref, TOL["f32"])
            assert_close("h_last", hn, h_ref, TOL["f32"])
        else:
            assert rc == ssm.SSM_ERR_HANDOFF
            assert np.isnan(yn).any() and np.isnan(hn).any()
    monkeypatch.delenv("SSM_SPLIT_SPIN_LIMIT", raising=False)


# ---- initial state h0 (resuming a sequence) ---------------------------------------

@pytest.mark.parametrize("Bs,L,ED,dtype,bidir", [(2, 300, 64, "f32", False), (1, 5000, 64, "f32", False),
                                                 (2, 257, 48, "bf16", False), (2, 200, 64, "f32", True)])
def test_initial_state(Bs, L, ED, dtype, bidir):
    log("case h0 Bs=%d L=%d ED=%d %s bidir=%s" % (Bs, L, ED, dtype, bidir))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L + 7)
    h0 = (0.5 * synth.normal(31, 8, (Bs, ED, 16))).astype(np.float32)
    y, h, _ = run_gpu(inp, bidir=bidir, want_h=True, h0=h0)
    y_ref, h_ref, _ = oracle.scan(**inp, h0=h0, bidir=bidir, want_h_last=True)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])


def test_resume_in_two_pieces():
    # scan [0, L1), then [L1, L) from the first piece's final state: the
    # concatenation matches the oracle's scan of the whole sequence
    log("case resume")
    Bs, L, ED, L1 = 2, 3000, 64, 1111
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=41)
    cut = lambda a, b: {k: (np.ascontiguousarray(v[:, a:b]) if k in ("x", "delta", "B", "C") else v)
                        for k, v in inp.items()}
    y1, h1, _ = run_gpu(cut(0, L1), want_h=True)
    y2, h2, _ = run_gpu(cut(L1, L), want_h=True, h0=h1.astype(np.float32))
    y_ref, h_ref, _ = oracle.scan(**inp, want_h_last=True)
    assert_close("y", np.concatenate([y1, y2], axis=1), y_ref, TOL["f32"])
    assert_close("h_last", h2, h_ref, TOL["f32"])


# ---- step-size pre-processing and output gate ------------------------------------

@pytest.mark.parametrize("Bs,L,ED,dtype,bidir", [(2, 300, 64, "f32", False), (2, 301, 40, "f32", False),
                                                 (2, 257, 64, "bf16", False), (2, 200, 64, "f32", True),
                                                 (1, 5000, 64, "f32", False), (1, 4500, 48, "bf16", False)])
def test_preprocessing_and_gate(Bs, L, ED, dtype, bidir):
    log("case options Bs=%d L=%d ED=%d %s bidir=%s" % (Bs, L, ED, dtype, bidir))
    inp, opts = options_inputs(Bs, L, ED, dtype, seed=L + ED)
    y, h, _ = run_gpu(inp, bidir=bidir, want_h=True, opts=opts)
    y_ref, h_ref, _ = oracle.scan(**inp, bidir=bidir, want_h_last=True, **opts)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])


def test_options_each_alone():
    inp, opts = options_inputs(2, 150, 32, "f32", seed=5)
    positive = synth.make_inputs(2, 150, 32, 16, "f32", seed=5)["delta"]   # log-uniform steps
    singles = {"dt_bias": dict(dt_bias=np.abs(opts["dt_bias"]) * 0.02),
               "dt_softplus": dict(dt_softplus=True),
               "dt_limit": dict(dt_limit=(0.01, 0.05)),
               "z": dict(z=opts["z"])}
    for key, one in singles.items():
        log("case option %s alone" % key)
        # raw steps only through softplus; otherwise positive steps (negative
        # raw steps make the state grow without bound)
        inp2 = inp if key == "dt_softplus" else dict(inp, delta=positive)
        y, h, _ = run_gpu(inp2, want_h=True, opts=one)
        y_ref, h_ref, _ = oracle.scan(**inp2, want_h_last=True, **one)
        assert_close("y", y, y_ref, TOL["f32"])
        assert_close("h_last", h, h_ref, TOL["f32"])


@pytest.mark.parametrize("Bs,L,ED", [(2, 0, 48), (0, 17, 48), (2, 17, 0), (3, 0, 21)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_inputs(Bs, L, ED, dtype):
    """Zero batch rows, steps or channels: nothing is scanned; over an empty
    sequence the forward state stays h0 (zero without it) and the reverse
    state is zero, as the oracle gives."""
    log("empty case Bs=%d L=%d ED=%d dtype=%s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=41)
    h0 = (0.5 * synth.normal(41, 9, (Bs, ED, 16))).astype(np.float32)
    for with_h0 in (False, True):
        h0v = h0 if with_h0 else None
        y, h, _ = run_gpu(inp, want_h=True, h0=h0v)
        y_ref, h_ref, _ = oracle.scan(**inp, h0=h0v, want_h_last=True)
        assert_close("y", y, y_ref, TOL[dtype])
        assert_close("h_last", h, h_ref, TOL["f32"])
        y, h, g = run_gpu(inp, bidir=True, want_h=True, want_g=True, h0=h0v)
        y_ref, h_ref, g_ref = oracle.scan(**inp, h0=h0v, bidir=True, want_h_last=True, want_g_first=True)
        assert_close("y bidir", y, y_ref, TOL[dtype])
        assert_close("h_last bidir", h, h_ref, TOL["f32"])
        assert_close("g_first", g, g_ref, TOL["f32"])

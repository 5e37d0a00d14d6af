"""Round checkpoints: ssm_scan_fwd_ckpt writes the state entering every
32-step round (checked against the oracle's state after the same prefix of
the sequence), and ssm_scan_bwd_ckpt, given them, skips its own forward sweep
(gradients checked against the oracle's adjoint, as the plain backward's)."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import (TOL, assert_close, assert_grads_close, log, options_inputs, run_gpu, run_gpu_bwd,
                         sample_channels, to_device, y_to_numpy)

pytestmark = pytest.mark.gpu


def run_fwd_ckpt(inp, h0=None, opts=None):
    import torch
    import state_space_model_selective_amd as ssm
    dev = torch.device("cuda:0")
    t = to_device(inp, dev)
    Bs, L, ED = inp["x"].shape
    ck = torch.full(ssm.ssm_scan_ckpt_shape(Bs, L, ED), float("nan"), dtype=torch.float32, device=dev)
    h0t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).to(dev)
    kw = dict(opts or {})
    if kw.get("dt_bias") is not None:
        kw["dt_bias"] = torch.from_numpy(np.ascontiguousarray(kw["dt_bias"], dtype=np.float32)).to(dev)
    y = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], h0=h0t, ckpt=ck, **kw)
    torch.cuda.synchronize()
    return y_to_numpy(y), ck.double().cpu().numpy()


def check_checkpoints(inp, rounds, chans, h0=None, opts=None, tol=TOL["f32"]):
    """Compare ckpt[b, r, e, :] with the oracle's state after 32 r steps for
    the sampled channels (ids b*ED + e) and rounds."""
    Bs, L, ED = inp["x"].shape
    y, ck = run_fwd_ckpt(inp, h0=h0, opts=opts)
    assert not np.isnan(ck[:, 1:, :ED]).any(), "a checkpoint was not written"
    assert not np.isnan(ck[:, 1:, ED:]).any(), "a padded channel's checkpoint was not written"
    assert np.all(ck[:, 1:, ED:] == 0.0), "padded channels keep their zero state"
    o = dict(opts or {})
    for r in rounds:
        t = 32 * r
        pre = {k: inp[k][:, :t] for k in ("x", "delta", "B", "C")}
        _, h, _ = oracle.scan(**pre, A=inp["A"], D=inp["D"], h0=h0, want_h_last=True, chans=chans,
                              dt_bias=o.get("dt_bias"), dt_softplus=o.get("dt_softplus", False),
                              dt_limit=o.get("dt_limit") or (-float("inf"), float("inf")))
        got = np.stack([ck[c // ED, r, c % ED] for c in chans])
        assert_close("ckpt round %d" % r, got, h, tol)
    return y


def plain_y(inp, h0=None, opts=None):
    y, _, _ = run_gpu(inp, h0=h0, opts=opts)
    return y


@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 200, 48, "f32"), (2, 257, 40, "bf16"), (3, 33, 20, "f32"),
                                           (2, 64, 130, "f32")])
def test_forward_checkpoints(Bs, L, ED, dtype):
    log("ckpt forward Bs=%d L=%d ED=%d %s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L)
    rounds = sorted({1, (L - 1) // 32, max(1, L // 64)})
    chans = sample_channels(Bs, ED, 12, seed=L)
    y = check_checkpoints(inp, [r for r in rounds if 1 <= r < (L + 31) // 32], chans)
    # writing checkpoints leaves the scan's output as it was, bit for bit
    np.testing.assert_array_equal(y, plain_y(inp))


def test_forward_checkpoints_one_round_writes_nothing():
    inp = synth.make_inputs(2, 31, 20, 16, "f32", seed=4)
    _, ck = run_fwd_ckpt(inp)
    assert ck.shape[1] == 1 and np.isnan(ck).all()


def test_forward_checkpoints_initial_state_and_options():
    inp, opts = options_inputs(2, 150, 48, "f32", seed=5)
    opts = {k: v for k, v in opts.items() if k != "z"}
    h0 = synth.normal(5, 79, (2, 48, 16))
    check_checkpoints(inp, [1, 2, 4], sample_channels(2, 48, 10, seed=5), h0=h0, opts=opts)


@pytest.mark.parametrize("Bs,L,ED", [(1, 16384, 64), (1, 9001, 32)])
def test_forward_checkpoints_split_sequence(Bs, L, ED):
    """Long sequences with few channel groups run split into chunks; a
    chunk's checkpoints take its entering state from the hand-off (rounds
    right after a chunk start as well as later ones)."""
    import state_space_model_selective_amd as ssm
    assert ssm.ssm_scan_workspace_bytes(Bs, L, ED, 16) > 0, "this shape is expected to split the sequence"
    log("ckpt split forward Bs=%d L=%d ED=%d" % (Bs, L, ED))
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=L)
    R = (L + 31) // 32
    rounds = sorted({1, 2, R // 7, R // 5 + 1, R // 3, R // 2, R // 2 + 1, (2 * R) // 3, R - 2, R - 1})
    check_checkpoints(inp, [r for r in rounds if 1 <= r < R], sample_channels(Bs, ED, 8, seed=L))


def check_bwd(Bs, L, ED, dtype="f32", seed=0, h0=False, **kw):
    log("ckpt bwd Bs=%d L=%d ED=%d %s seed=%d" % (Bs, L, ED, dtype, seed))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=seed)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=seed)
    h = synth.normal(seed, 79, (Bs, ED, 16)) if h0 else None
    got = run_gpu_bwd(inp, dy, h0=h, want_dh0=True, use_ckpt=True, **kw)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h, dh_last=kw.get("dh_last"))
    assert_grads_close(got, ref, dtype)
    return inp, dy, got


@pytest.mark.parametrize("L", [1, 31, 33, 64, 200, 1009])
def test_backward_with_checkpoints(L):
    check_bwd(2, L, 48, seed=L)


def test_backward_with_checkpoints_bf16_and_state():
    check_bwd(2, 300, 96, dtype="bf16", seed=5, h0=True)


def test_backward_with_checkpoints_final_state_gradient():
    check_bwd(2, 150, 40, seed=6, dh_last=synth.normal(6, 81, (2, 40, 16)))


def test_backward_with_checkpoints_matches_plain_backward():
    inp = synth.make_inputs(2, 257, 80, 16, "f32", seed=7)
    dy = synth.make_output_grad(2, 257, 80, "f32", seed=7)
    a = run_gpu_bwd(inp, dy, want_dh0=True, use_ckpt=True)
    b = run_gpu_bwd(inp, dy, want_dh0=True)
    for k in a:
        assert_close(k, a[k], b[k], 2e-5)


def test_backward_with_checkpoints_options_and_gate():
    inp, opts = options_inputs(2, 200, 48, "f32", seed=8)
    dy = synth.make_output_grad(2, 200, 48, "f32", seed=8)
    got = run_gpu_bwd(inp, dy, want_dh0=True, use_ckpt=True, **opts)
    ref = oracle.scan_bwd(**inp, dy=dy, **{k: v for k, v in opts.items()})
    assert_grads_close(got, ref, "f32")


def test_backward_with_checkpoints_split_sequence():
    """The backward splits this sequence too (its own chunks); the forward's
    checkpoints come from a split forward."""
    Bs, L, ED = 1, 9001, 32
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=9)
    dy = synth.make_output_grad(Bs, L, ED, "f32", seed=9)
    got = run_gpu_bwd(inp, dy, want_dh0=True, use_ckpt=True)
    ref = oracle.scan_bwd(**inp, dy=dy)
    assert_grads_close(got, ref, "f32")


# ---- the bidirectional scan: the forward direction's checkpoints ------------

def run_bidir_fwd_ckpt(inp, h0=None, g0=None, opts=None):
    import torch
    import state_space_model_selective_amd as ssm
    dev = torch.device("cuda:0")
    t = to_device(inp, dev)
    Bs, L, ED = inp["x"].shape
    ck = torch.full(ssm.ssm_scan_ckpt_shape(Bs, L, ED), float("nan"), dtype=torch.float32, device=dev)
    st = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    kw = dict(opts or {})
    if kw.get("dt_bias") is not None:
        kw["dt_bias"] = st(kw["dt_bias"])
    y = ssm.ssm_scan_bidir_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], h0=st(h0), g0=st(g0), ckpt=ck,
                               **kw)
    torch.cuda.synchronize()
    return y_to_numpy(y), ck.double().cpu().numpy()


@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 200, 48, "f32"), (2, 257, 40, "bf16"), (1, 9001, 32, "f32"),
                                           (1, 3000, 64, "f32")])
def test_bidir_forward_checkpoints(Bs, L, ED, dtype):
    """The forward direction's states after each prefix, from h0, whatever
    the reverse direction starts from; split shapes take their corrections
    in the join kernel. y is the plain bidirectional forward's, bit for bit."""
    log("ckpt bidir forward Bs=%d L=%d ED=%d %s" % (Bs, L, ED, dtype))
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=L + 1)
    h0 = synth.normal(L, 79, (Bs, ED, 16))
    g0 = synth.normal(L, 80, (Bs, ED, 16))
    y, ck = run_bidir_fwd_ckpt(inp, h0=h0, g0=g0)
    R = (L + 31) // 32
    assert not np.isnan(ck[:, 1:]).any(), "a checkpoint was not written"
    chans = sample_channels(Bs, ED, 8, seed=L)
    for r in sorted({1, 2, R // 3, R // 2 + 1, R - 1}):
        if not 1 <= r < R:
            continue
        pre = {k: inp[k][:, :32 * r] for k in ("x", "delta", "B", "C")}
        _, h, _ = oracle.scan(**pre, A=inp["A"], D=inp["D"], h0=h0, want_h_last=True, chans=chans)
        got = np.stack([ck[c // ED, r, c % ED] for c in chans])
        assert_close("ckpt round %d" % r, got, h, TOL["f32"])
    y0, _, _ = run_gpu(inp, bidir=True, h0=h0, g0=g0)
    np.testing.assert_array_equal(y, y0)


@pytest.mark.parametrize("Bs,L,ED,dtype", [(2, 200, 48, "f32"), (2, 300, 96, "bf16"), (1, 3000, 64, "f32")])
def test_bidir_backward_with_checkpoints(Bs, L, ED, dtype):
    log("ckpt bidir bwd Bs=%d L=%d ED=%d %s" % (Bs, L, ED, dtype))
    seed = L + ED + 3
    inp = synth.make_inputs(Bs, L, ED, 16, dtype, seed=seed)
    dy = synth.make_output_grad(Bs, L, ED, dtype, seed=seed)
    h0 = synth.normal(seed, 79, (Bs, ED, 16))
    kw = dict(g0=synth.normal(seed, 81, (Bs, ED, 16)), dg_first=synth.normal(seed, 82, (Bs, ED, 16)))
    dhl = synth.normal(seed, 80, (Bs, ED, 16))
    got = run_gpu_bwd(inp, dy, h0=h0, want_dh0=True, bidir=True, dh_last=dhl, want_dg0=True, use_ckpt=True, **kw)
    ref = oracle.scan_bwd(**inp, dy=dy, h0=h0, bidir=True, dh_last=dhl, **kw)
    assert_grads_close(got, ref, dtype)


def test_bidir_backward_with_checkpoints_options_and_gate():
    inp, opts = options_inputs(2, 200, 48, "f32", seed=11)
    dy = synth.make_output_grad(2, 200, 48, "f32", seed=11)
    got = run_gpu_bwd(inp, dy, want_dh0=True, bidir=True, use_ckpt=True, **opts)
    ref = oracle.scan_bwd(**inp, dy=dy, bidir=True, **opts)
    assert_grads_close(got, ref, "f32")

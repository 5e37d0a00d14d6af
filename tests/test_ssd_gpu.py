"""GPU parity of the multi-head (SSD) scan (ssm_ssd_fwd) against the oracle
(oracle.ssd) on the same seeded inputs."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import TOL, assert_close, log, run_gpu_ssd, to_device

pytestmark = pytest.mark.gpu


def check(Bs, L, H, G, N, dtype="f32", seed=0, h0=False, D_none=False):
    log("ssd case Bs=%d L=%d H=%d G=%d N=%d dtype=%s seed=%d h0=%s D_none=%s" % (Bs, L, H, G, N, dtype, seed, h0,
                                                                               D_none))
    inp = synth.make_ssd_inputs(Bs, L, H, 64, G, N, dtype, seed=seed)
    h = synth.normal(seed, 93, (Bs, H, 64, N)) if h0 else None
    y, hl = run_gpu_ssd(inp, h0=h, want_h=True, D_none=D_none)
    y_ref, h_ref, _ = oracle.ssd(**(dict(inp, D=None) if D_none else inp), h0=h, want_h_last=True)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", hl, h_ref, TOL["f32"])


def test_small():
    check(2, 64, 4, 1, 64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 100, 400])
def test_sequence_lengths(L, dtype):
    check(2, L, 2, 1, 128, dtype=dtype, seed=L)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_128_and_groups(dtype):
    check(2, 150, 8, 2, 128, dtype=dtype, seed=3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_groups_64(dtype):
    check(3, 70, 6, 3, 64, dtype=dtype, seed=4)


def test_bf16():
    check(2, 200, 4, 1, 128, dtype="bf16", seed=5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_initial_state(dtype):
    check(2, 90, 4, 2, 128, dtype=dtype, seed=6, h0=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_D(dtype):
    check(1, 50, 2, 1, 64, dtype=dtype, seed=7, D_none=True)


def test_bf16_long_state_accuracy():
    # 128 chunks: the bf16 operand splitting keeps the carried state at float32 accuracy
    check(1, 4096, 2, 1, 128, dtype="bf16", seed=9, h0=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeatable_bits(dtype):
    inp = synth.make_ssd_inputs(2, 77, 4, 64, 1, 128, dtype, seed=8)
    a, ha = run_gpu_ssd(inp, want_h=True)
    b, hb = run_gpu_ssd(inp, want_h=True)
    assert np.array_equal(a, b) and np.array_equal(ha, hb)


@pytest.mark.parametrize("name", sorted(synth.SSD_WORKLOADS))
def test_workloads(name):
    w = synth.SSD_WORKLOADS[name]
    bidir = w.get("bidir", False)
    log("ssd workload %s" % name)
    inp = synth.make_ssd_inputs(w["Bs"], w["L"], w["H"], w["P"], w["G"], w["N"], w["dtype"], seed=0)
    out = run_gpu_ssd(inp, want_h=True, want_g=bidir, bidir=bidir)
    ref = oracle.ssd(**inp, bidir=bidir, want_h_last=True, want_g_first=bidir)
    assert_close("y", out[0], ref[0], TOL[w["dtype"]])
    assert_close("h_last", out[1], ref[1], TOL["f32"])
    if bidir:
        assert_close("g_first", out[2], ref[2], TOL["f32"])


def check_bidir(Bs, L, H, G, N, dtype="f32", seed=0, h0=False, D_none=False):
    log("ssd bidir case Bs=%d L=%d H=%d G=%d N=%d dtype=%s seed=%d h0=%s D_none=%s" % (Bs, L, H, G, N, dtype, seed,
                                                                                     h0, D_none))
    inp = synth.make_ssd_inputs(Bs, L, H, 64, G, N, dtype, seed=seed)
    h = synth.normal(seed, 94, (Bs, H, 64, N)) if h0 else None
    y, hl, gf = run_gpu_ssd(inp, h0=h, want_h=True, want_g=True, D_none=D_none, bidir=True)
    ref_inp = dict(inp, D=None) if D_none else inp
    y_ref, h_ref, g_ref = oracle.ssd(**ref_inp, h0=h, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", hl, h_ref, TOL["f32"])
    assert_close("g_first", gf, g_ref, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 31, 32, 33, 100, 400])
def test_bidirectional_sequence_lengths(L, dtype):
    check_bidir(2, L, 2, 1, 128, dtype=dtype, seed=L + 50)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidirectional_groups_and_state_64(dtype):
    check_bidir(3, 70, 6, 3, 64, dtype=dtype, seed=51)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidirectional_initial_state_and_no_D(dtype):
    check_bidir(2, 90, 4, 2, 128, dtype=dtype, seed=52, h0=True, D_none=True)


def test_bidirectional_long_bf16():
    check_bidir(1, 4096, 2, 1, 128, dtype="bf16", seed=53, h0=True)


def test_bidirectional_workspace_checks():
    import torch
    import state_space_model_selective_amd as ssm
    inp = synth.make_ssd_inputs(1, 40, 2, 64, 1, 64, "bf16", seed=54)
    t = to_device(inp, torch.device("cuda:0"))
    need = ssm.ssm_ssd_bidir_workspace_bytes(1, 40, 2, 64, ssm.SSM_BF16)
    assert need >= 1 * 40 * 2 * 64 * 4
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ssm.SSMError) as e:
        ssm.ssm_ssd_bidir_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], workspace=small)
    assert e.value.status == ssm.SSM_ERR_WORKSPACE


def check_options(Bs, L, H, G, N, dtype, seed, bidir=False, bias=True, softplus=True, limit=(0.02, 0.3),
                  gate=True, h0=False):
    log("ssd options case Bs=%d L=%d H=%d G=%d N=%d dtype=%s seed=%d bidir=%s bias=%s softplus=%s limit=%s "
        "gate=%s h0=%s" % (Bs, L, H, G, N, dtype, seed, bidir, bias, softplus, limit, gate, h0))
    inp = synth.make_ssd_inputs(Bs, L, H, 64, G, N, dtype, seed=seed)
    opts = {}
    if bias:
        nb = synth.normal(seed, 99, (H,))
        if softplus or (limit is not None and limit[0] > 0):
            # mostly negative: dt + bias < 0 for many steps, which softplus or the clamp maps back
            opts["dt_bias"] = (nb * 0.5 - 1.5).astype(np.float32)
        else:
            # the bias alone must keep the step positive (a negative step grows the state
            # without bound: the overflow regime outside the contract)
            opts["dt_bias"] = (np.abs(nb) * 0.05).astype(np.float32)
    if softplus:
        opts["dt_softplus"] = True
    if limit is not None:
        opts["dt_limit"] = limit
    if gate:
        z = synth.normal(seed, 100, (Bs, L, H, 64))
        opts["z"] = synth.to_bf16(z) if dtype == "bf16" else z
    h = synth.normal(seed, 101, (Bs, H, 64, N)) if h0 else None
    out = run_gpu_ssd(inp, h0=h, want_h=True, want_g=bidir, bidir=bidir, opts=opts)
    ref = oracle.ssd(**inp, h0=h, bidir=bidir, want_h_last=True, want_g_first=bidir, **opts)
    assert_close("y", out[0], ref[0], TOL[dtype])
    assert_close("h_last", out[1], ref[1], TOL["f32"])
    if bidir:
        assert_close("g_first", out[2], ref[2], TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 33, 200])
def test_options_all(L, dtype):
    check_options(2, L, 4, 2, 128, dtype, seed=60 + L)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_options_bidirectional(dtype):
    check_options(2, 150, 4, 1, 128, dtype, seed=61, bidir=True, h0=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_options_state_64_bidirectional_ragged(dtype):
    check_options(1, 77, 2, 1, 64, dtype, seed=62, bidir=True)


@pytest.mark.parametrize("which", ["bias", "softplus", "limit", "gate"])
def test_options_one_at_a_time(which):
    # each option alone (the others off), bf16 and f32 alternating
    kw = dict(bias=which == "bias", softplus=which == "softplus", limit=(0.02, 0.3) if which == "limit" else None,
              gate=which == "gate")
    check_options(2, 70, 4, 1, 128, "bf16" if which in ("bias", "gate") else "f32", seed=63, **kw)


@pytest.mark.parametrize("Bs,L", [(2, 0), (0, 40)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_inputs(Bs, L, dtype):
    """No batch rows or no steps: nothing is scanned; the forward state stays
    h0 and the reverse state is zero, as the oracle gives."""
    log("ssd empty case Bs=%d L=%d dtype=%s" % (Bs, L, dtype))
    H, P, G, N = 4, 64, 1, 64
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, dtype, seed=43)
    h0 = (0.5 * synth.normal(43, 9, (Bs, H, P, N))).astype(np.float32)
    y, h = run_gpu_ssd(inp, h0=h0, want_h=True)
    y_ref, h_ref, _ = oracle.ssd(**inp, h0=h0, want_h_last=True)
    assert_close("y", y, y_ref, TOL[dtype])
    assert_close("h_last", h, h_ref, TOL["f32"])
    y, h, g = run_gpu_ssd(inp, h0=h0, want_h=True, bidir=True, want_g=True)
    y_ref, h_ref, g_ref = oracle.ssd(**inp, h0=h0, bidir=True, want_h_last=True, want_g_first=True)
    assert_close("y bidir", y, y_ref, TOL[dtype])
    assert_close("h_last bidir", h, h_ref, TOL["f32"])
    assert_close("g_first", g, g_ref, TOL["f32"])


# ---- split sequences: fewer (batch row, head) pairs than compute units -------
# Each sweep is cut into ranges of whole chunks: a first pass forms every
# range's end state from zero, a small kernel folds them into the state
# entering each range (from h0 / g0), and every range then runs from it.

@pytest.mark.parametrize("Bs,L,H,G,N,dtype,bidir", [
    (1, 3000, 3, 1, 128, "f32", False), (1, 3000, 3, 1, 128, "bf16", False), (2, 2100, 2, 2, 64, "bf16", False),
    (1, 2600, 2, 1, 64, "f32", False), (1, 3000, 3, 1, 128, "f32", True), (1, 2600, 4, 2, 128, "bf16", True)])
def test_split_sequence(Bs, L, H, G, N, dtype, bidir):
    import state_space_model_selective_amd as ssm
    code = ssm.SSM_F32 if dtype == "f32" else ssm.SSM_BF16
    need = (ssm.ssm_ssd_bidir_workspace_bytes if bidir else ssm.ssm_ssd_workspace_bytes)(Bs, L, H, 64, code)
    plain = -(-Bs * L * H * 64 * 4 // 256) * 256 if (bidir and dtype == "bf16") else 0
    assert need > plain, "this shape is expected to split its sequences"
    seed = L + H + N
    log("ssd split case Bs=%d L=%d H=%d G=%d N=%d %s bidir=%s" % (Bs, L, H, G, N, dtype, bidir))
    inp = synth.make_ssd_inputs(Bs, L, H, 64, G, N, dtype, seed=seed)
    h0 = synth.normal(seed, 95, (Bs, H, 64, N))
    g0 = synth.normal(seed, 96, (Bs, H, 64, N)) if bidir else None
    out = run_gpu_ssd(inp, h0=h0, want_h=True, want_g=bidir, bidir=bidir, g0=g0)
    ref = oracle.ssd(**inp, h0=h0, g0=g0, bidir=bidir, want_h_last=True, want_g_first=bidir)
    assert_close("y", out[0], ref[0], TOL[dtype])
    assert_close("h_last", out[1], ref[1], TOL["f32"])
    if bidir:
        assert_close("g_first", out[2], ref[2], TOL["f32"])


@pytest.mark.parametrize("dtype,bidir", [("f32", False), ("bf16", False), ("bf16", True)])
def test_split_sequence_with_options(dtype, bidir):
    check_options(1, 2500, 2, 1, 128, dtype, seed=64, bidir=bidir, h0=True)

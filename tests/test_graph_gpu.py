"""The entry points under HIP graph capture (torch.cuda.graph): each call is
captured once and replayed several times, with the outputs overwritten and
other eager work and synchronisations between the replays; every replay must
reproduce the eager result bit for bit. The captured calls include the
kernel that clears the split-sequence workspace (no memset node), the
backward's reduction kernels and the bidirectional calls' workspaces."""
import numpy as np
import pytest

import synth
from parity_util import log, to_device

pytestmark = pytest.mark.gpu


def replay_check(name, fn, outs, reps=4):
    import torch
    log("graph case %s" % name)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up off the default stream, as capture wants
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    fn()  # the eager result
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for r in ref:
        assert bool(torch.isfinite(r.float()).all()), "eager result of %s is not finite" % name
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for i in range(reps):
        for o in outs:
            o.fill_(float("nan"))
        noise = torch.randn(1 << 20, device=outs[0].device)
        float(noise.abs().sum())  # eager work and a synchronisation between replays
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), "%s: replay %d differs from the eager result in output %d" % (name, i, k)


def test_forward_split_sequence_graph():
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 1, 8192, 64, 16
    need = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, ssm.SSM_F32, False)
    assert need > 0, "this shape should take the split-sequence path"
    dev = torch.device("cuda:0")
    t = to_device(synth.make_inputs(Bs, L, ED, N, "f32", seed=70), dev)
    y = torch.empty_like(t["x"])
    h = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    replay_check("forward, split sequence", lambda: ssm.ssm_scan_fwd(
        t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=y, h_last=h, workspace=ws), [y, h])


def test_bidirectional_bf16_graph():
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 2, 600, 128, 16
    need = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, ssm.SSM_BF16, True)
    dev = torch.device("cuda:0")
    t = to_device(synth.make_inputs(Bs, L, ED, N, "bf16", seed=71), dev)
    y = torch.empty_like(t["x"])
    gf = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    replay_check("bidirectional bf16", lambda: ssm.ssm_scan_bidir_fwd(
        t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=y, g_first=gf, workspace=ws if need else None),
        [y, gf])


def test_backward_graph():
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 2, 300, 64, 16
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=72)
    t = to_device(dict(inp, dy=synth.make_output_grad(Bs, L, ED, "f32", seed=72)), dev)
    out = {"dx": torch.empty_like(t["x"]), "ddelta": torch.empty_like(t["x"]), "dA": torch.empty_like(t["A"]),
           "dB": torch.empty_like(t["B"]), "dC": torch.empty_like(t["B"]),
           "dD": torch.empty((ED,), dtype=torch.float32, device=dev)}
    need = ssm.ssm_scan_bwd_workspace_bytes(Bs, L, ED, N, ssm.SSM_F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    replay_check("backward", lambda: ssm.ssm_scan_bwd(
        t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dy"], out=out, workspace=ws),
        [out[k] for k in ("dx", "ddelta", "dA", "dB", "dC", "dD")])


def test_multi_head_bidirectional_options_graph():
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, H, P, G, N = 1, 200, 4, 64, 1, 128
    dev = torch.device("cuda:0")
    t = to_device(synth.make_ssd_inputs(Bs, L, H, P, G, N, "bf16", seed=73), dev)
    z = to_device({"z": synth.to_bf16(synth.normal(73, 100, (Bs, L, H, P)))}, dev)["z"]
    bias = torch.from_numpy(np.ascontiguousarray(synth.normal(73, 99, (H,)) * 0.5 - 1.0, dtype=np.float32)).to(dev)
    y = torch.empty_like(t["x"])
    h = torch.empty((Bs, H, P, N), dtype=torch.float32, device=dev)
    need = ssm.ssm_ssd_bidir_workspace_bytes(Bs, L, H, P, ssm.SSM_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    replay_check("multi-head bidirectional bf16 with options", lambda: ssm.ssm_ssd_bidir_fwd(
        t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], y=y, h_last=h, workspace=ws, dt_bias=bias,
        dt_softplus=True, dt_limit=(0.01, 0.5), z=z), [y, h])


def test_bidirectional_backward_bf16_graph():
    # two backward launches (the second adding to the first's float32 dx and
    # ddelta in the workspace) and the reductions over both directions
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 2, 300, 64, 16
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(Bs, L, ED, N, "bf16", seed=74)
    t = to_device(dict(inp, dy=synth.make_output_grad(Bs, L, ED, "bf16", seed=74)), dev)
    out = {"dx": torch.empty_like(t["x"]), "ddelta": torch.empty_like(t["x"]), "dA": torch.empty_like(t["A"]),
           "dB": torch.empty_like(t["B"]), "dC": torch.empty_like(t["B"]),
           "dD": torch.empty((ED,), dtype=torch.float32, device=dev)}
    need = ssm.ssm_scan_bidir_bwd_workspace_bytes(Bs, L, ED, N, ssm.SSM_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    replay_check("bidirectional backward bf16", lambda: ssm.ssm_scan_bidir_bwd(
        t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dy"], out=out, workspace=ws),
        [out[k] for k in ("dx", "ddelta", "dA", "dB", "dC", "dD")])


def test_bidirectional_split_sequence_graph():
    # the split bidirectional scan: the chunk kernel and the join kernel
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 1, 6000, 64, 16
    need = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, ssm.SSM_F32, True)
    assert need > 0, "this shape should split the bidirectional scan"
    dev = torch.device("cuda:0")
    t = to_device(synth.make_inputs(Bs, L, ED, N, "f32", seed=75), dev)
    y = torch.empty_like(t["x"])
    h = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)
    gf = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    replay_check("bidirectional, split sequence", lambda: ssm.ssm_scan_bidir_fwd(
        t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=y, h_last=h, g_first=gf, workspace=ws), [y, h, gf])


@pytest.mark.parametrize("bidir", [False, True])
def test_backward_split_sweep_graph(bidir):
    # the chunk-aggregate kernel, the chunked backward and the reductions
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 1, 4000, 48, 16
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=76)
    t = to_device(dict(inp, dy=synth.make_output_grad(Bs, L, ED, "f32", seed=76)), dev)
    out = {"dx": torch.empty_like(t["x"]), "ddelta": torch.empty_like(t["x"]), "dA": torch.empty_like(t["A"]),
           "dB": torch.empty_like(t["B"]), "dC": torch.empty_like(t["B"]),
           "dD": torch.empty((ED,), dtype=torch.float32, device=dev),
           "dh0": torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)}
    fn = ssm.ssm_scan_bidir_bwd if bidir else ssm.ssm_scan_bwd
    need = (ssm.ssm_scan_bidir_bwd_workspace_bytes if bidir else ssm.ssm_scan_bwd_workspace_bytes)(
        Bs, L, ED, N, ssm.SSM_F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    replay_check("backward, split sweep, bidir=%s" % bidir, lambda: fn(
        t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dy"], out=out, workspace=ws, want_dh0=True),
        [out[k] for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dh0")])


@pytest.mark.parametrize("bidir", [False, True])
def test_multi_head_split_sequence_graph(bidir):
    # the aggregate pass, the join kernel and the ranges (the bidirectional
    # scan with its reverse sweep in a launch of its own)
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, H, P, G, N = 1, 2600, 2, 64, 1, 128
    dtype = "bf16" if bidir else "f32"
    code = ssm.SSM_BF16 if bidir else ssm.SSM_F32
    need = (ssm.ssm_ssd_bidir_workspace_bytes if bidir else ssm.ssm_ssd_workspace_bytes)(Bs, L, H, P, code)
    assert need > (Bs * L * H * P * 4 if bidir else 0), "this shape should split its sequences"
    dev = torch.device("cuda:0")
    t = to_device(synth.make_ssd_inputs(Bs, L, H, P, G, N, dtype, seed=77), dev)
    y = torch.empty_like(t["x"])
    h = torch.empty((Bs, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    fn = ssm.ssm_ssd_bidir_fwd if bidir else ssm.ssm_ssd_fwd
    replay_check("multi-head split sequence, bidir=%s" % bidir, lambda: fn(
        t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], y=y, h_last=h, workspace=ws), [y, h])


@pytest.mark.parametrize("bidir", [False, True])
def test_training_step_pair_graph(bidir):
    """The forward that keeps the round states and the backward that reads
    them, captured together (split sequences, so the forward's workspace
    clear and the backward's aggregate pass are in the graph too)."""
    import torch
    import state_space_model_selective_amd as ssm
    Bs, L, ED, N = 1, 8192, 64, 16
    dev = torch.device("cuda:0")
    t = to_device(synth.make_inputs(Bs, L, ED, N, "f32", seed=72), dev)
    dy = to_device(dict(dy=synth.make_output_grad(Bs, L, ED, "f32", seed=72)), dev)["dy"]
    y = torch.empty_like(t["x"])
    ck = torch.empty(ssm.ssm_scan_ckpt_shape(Bs, L, ED), dtype=torch.float32, device=dev)
    fneed = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, ssm.SSM_F32, bidir)
    fws = torch.empty(max(fneed, 1), dtype=torch.uint8, device=dev) if fneed else None
    bneed = (ssm.ssm_scan_bidir_bwd_workspace_bytes if bidir else ssm.ssm_scan_bwd_workspace_bytes)(
        Bs, L, ED, N, ssm.SSM_F32)
    bws = torch.empty(bneed, dtype=torch.uint8, device=dev)
    out = {k: torch.empty_like(v) for k, v in (("dx", t["x"]), ("ddelta", t["x"]), ("dA", t["A"]), ("dB", t["B"]),
                                               ("dC", t["C"]))}
    out["dD"] = torch.empty((ED,), dtype=torch.float32, device=dev)
    args = (t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"])
    fwd = ssm.ssm_scan_bidir_fwd if bidir else ssm.ssm_scan_fwd
    bwd = ssm.ssm_scan_bidir_bwd if bidir else ssm.ssm_scan_bwd

    def step():
        fwd(*args, y=y, workspace=fws, ckpt=ck)
        bwd(*args, dy, out=out, workspace=bws, ckpt=ck)

    # (the checkpoints are an intermediate: their round 0 is never written)
    replay_check("training step, bidir=%s" % bidir, step, [y] + [out[k] for k in sorted(out)])

"""Helpers for GPU parity tests: run the HIP path through the binding, run
the oracle on the same buffers, and compare under the stated tolerance

    pass  iff  max_i ( |y_i - y_ref_i| - tol * (1 + |y_ref_i|) ) <= 0,

tol = 1e-4 for float32 outputs and 2e-2 for bfloat16 outputs (float32 state
and accumulation in both cases)."""
import sys

import numpy as np

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp, dev):
    import torch
    out = {}
    for k, v in inp.items():
        if not v.flags.writeable:
            v = v.copy()  # torch wants writable host memory
        if v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(v).to(dev)
    return out


def y_to_numpy(y):
    import torch
    if y.dtype == torch.bfloat16:
        return y.float().cpu().numpy().astype(np.float64)
    return y.double().cpu().numpy()


def run_gpu(inp, bidir=False, want_h=False, want_g=False, stream=None, D_none=False, h0=None, opts=None, g0=None):
    import torch
    import state_space_model_selective_amd as ssm
    dev = torch.device("cuda:0")
    t = to_device(inp, dev)
    Bs, L, ED = inp["x"].shape
    N = inp["A"].shape[1]
    h = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device=dev) if want_h else None
    g = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device=dev) if want_g else None
    D = None if D_none else t["D"]
    h0t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).to(dev)
    kw = {}
    if opts:
        kw = dict(opts)
        if kw.get("dt_bias") is not None:
            kw["dt_bias"] = torch.from_numpy(np.ascontiguousarray(kw["dt_bias"], dtype=np.float32)).to(dev)
        if kw.get("z") is not None:
            kw["z"] = to_device({"z": kw["z"]}, dev)["z"]
    if bidir:
        g0t = None if g0 is None else torch.from_numpy(np.ascontiguousarray(g0, dtype=np.float32)).to(dev)
        y = ssm.ssm_scan_bidir_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D, h_last=h, g_first=g,
                                   stream=stream, h0=h0t, g0=g0t, **kw)
    else:
        y = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D, h_last=h, stream=stream, h0=h0t, **kw)
    torch.cuda.synchronize()
    return (y_to_numpy(y), None if h is None else h.double().cpu().numpy(),
            None if g is None else g.double().cpu().numpy())


def excess(got, ref, tol):
    return np.abs(got - ref) - tol * (1.0 + np.abs(ref))


def assert_close(name, got, ref, tol, chunk_hint=None):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        log("  %s: empty %s" % (name, ref.shape))
        return 0.0
    assert np.all(np.isfinite(got)), "%s has non-finite values" % name
    ex = excess(got, ref, tol)
    i = np.unravel_index(np.argmax(ex), ex.shape)
    worst = float(ex[i])
    rel = float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))
    log("  %s: max |d|/(1+|ref|) = %.3e (tol %.0e) at %s" % (name, rel, tol, tuple(int(v) for v in i)))
    assert worst <= 0.0, "%s: tolerance exceeded by %.3e at index %s (got %r, ref %r)" % (
        name, worst, tuple(int(v) for v in i), float(got[i]), float(ref[i]))
    return rel


def sample_channels(Bs, ED, count, seed=0):
    """Channel ids b*ED + e: both ends, and a seeded spread in between."""
    rng = np.random.default_rng(seed)
    n = Bs * ED
    pick = {0, n - 1, ED - 1, min(ED, n - 1), n // 2}
    pick.update(int(v) for v in rng.integers(0, n, size=max(0, count - len(pick))))
    return np.array(sorted(pick), dtype=np.int64)


def gather_channels(y, chans, ED):
    """y (Bs, L, ED) -> (len(chans), L) in the oracle's channel-major order."""
    b, e = np.divmod(chans, ED)
    return y[b, :, e]


def run_gpu_bwd(inp, dy, h0=None, D_none=False, want_dD=True, want_dh0=False, stream=None, bidir=False,
                dt_bias=None, dt_softplus=False, dt_limit=None, z=None, dh_last=None, g0=None, dg_first=None,
                want_dg0=False, use_ckpt=False):
    """ssm_scan_bwd (bidir: ssm_scan_bidir_bwd) on the GPU; every gradient as
    a float64 numpy array. dt_bias (numpy, float32) / dt_softplus / dt_limit
    are the step-size options; with dt_bias the result holds ddt_bias; z (like
    x) is the output gate, and the result then holds dz. use_ckpt: run the
    forward (bidir: the bidirectional forward) with round checkpoints
    (NaN-filled first) and pass them to the backward."""
    import torch
    import state_space_model_selective_amd as ssm
    dev = torch.device("cuda:0")
    t = to_device(dict(inp, dy=dy), dev)
    h0t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).to(dev)
    # outputs start as NaN so that an element the kernels never write shows
    out = {}
    for k, ref in (("dx", t["x"]), ("ddelta", t["x"]), ("dA", t["A"]), ("dB", t["B"]), ("dC", t["B"])):
        out[k] = torch.full_like(ref, float("nan"))
    Bs, L, ED = inp["x"].shape
    N = inp["A"].shape[1]
    if want_dD:
        out["dD"] = torch.full((ED,), float("nan"), dtype=torch.float32, device=dev)
    if want_dh0:
        out["dh0"] = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device=dev)
    bias = None
    if dt_bias is not None:
        bias = torch.from_numpy(np.ascontiguousarray(dt_bias, dtype=np.float32)).to(dev)
        out["ddt_bias"] = torch.full((ED,), float("nan"), dtype=torch.float32, device=dev)
    zt = None
    if z is not None:
        zt = to_device(dict(z=z), dev)["z"]
        out["dz"] = torch.full_like(t["x"], float("nan"))
    st = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    kw = dict(dh_last=st(dh_last))
    if bidir:
        kw.update(g0=st(g0), dg_first=st(dg_first), want_dg0=want_dg0)
        if want_dg0:
            out["dg0"] = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device=dev)
    if use_ckpt:
        ck = torch.full(ssm.ssm_scan_ckpt_shape(Bs, L, ED), float("nan"), dtype=torch.float32, device=dev)
        fargs = (t["x"], t["delta"], t["A"], t["B"], t["C"], None if D_none else t["D"])
        fkw = dict(h0=h0t, dt_bias=bias, dt_softplus=dt_softplus, dt_limit=dt_limit, z=zt, ckpt=ck, stream=stream)
        if bidir:
            ssm.ssm_scan_bidir_fwd(*fargs, g0=kw["g0"], **fkw)
        else:
            ssm.ssm_scan_fwd(*fargs, **fkw)
        kw["ckpt"] = ck
    fn = ssm.ssm_scan_bidir_bwd if bidir else ssm.ssm_scan_bwd
    res = fn(t["x"], t["delta"], t["A"], t["B"], t["C"], None if D_none else t["D"], t["dy"],
             h0=h0t, want_dD=want_dD, want_dh0=want_dh0, out=out, stream=stream, dt_bias=bias,
             dt_softplus=dt_softplus, dt_limit=dt_limit, z=zt, **kw)
    torch.cuda.synchronize()
    return {k: y_to_numpy(v) for k, v in res.items()}


def assert_grads_close(got, ref, dtype):
    """Every gradient the GPU returned against the oracle's. dx, ddelta, dB,
    dC and dz carry the inputs' dtype; dA, dD, dh0, dg0 and ddt_bias are
    float32."""
    for k, v in got.items():
        tol = TOL[dtype] if k in ("dx", "ddelta", "dB", "dC", "dz") else TOL["f32"]
        assert_close(k, v, ref[k], tol)


def run_gpu_ssd(inp, h0=None, want_h=False, D_none=False, stream=None, bidir=False, want_g=False, opts=None,
                g0=None):
    """ssm_ssd_fwd (or ssm_ssd_bidir_fwd) on the GPU: (y, h_last) as float64
    numpy arrays, and g_first as a third value for the bidirectional scan.
    opts: dt_bias / dt_softplus / dt_limit / z as numpy values or None."""
    import torch
    import state_space_model_selective_amd as ssm
    dev = torch.device("cuda:0")
    t = to_device(inp, dev)
    Bs, L, H, P = inp["x"].shape
    N = inp["B"].shape[3]
    h = torch.full((Bs, H, P, N), float("nan"), dtype=torch.float32, device=dev) if want_h else None
    gf = torch.full((Bs, H, P, N), float("nan"), dtype=torch.float32, device=dev) if want_g else None
    h0t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).to(dev)
    y = torch.full_like(t["x"], float("nan"))
    D = None if D_none else t["D"]
    kw = {}
    if opts:
        kw = dict(opts)
        if kw.get("dt_bias") is not None:
            kw["dt_bias"] = torch.from_numpy(np.ascontiguousarray(kw["dt_bias"], dtype=np.float32)).to(dev)
        if kw.get("z") is not None:
            kw["z"] = to_device({"z": kw["z"]}, dev)["z"]
    if bidir:
        g0t = None if g0 is None else torch.from_numpy(np.ascontiguousarray(g0, dtype=np.float32)).to(dev)
        ssm.ssm_ssd_bidir_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D, y=y, h_last=h, g_first=gf, h0=h0t,
                              g0=g0t, stream=stream, **kw)
    else:
        ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D, y=y, h_last=h, h0=h0t, stream=stream, **kw)
    torch.cuda.synchronize()
    out = (y_to_numpy(y), (None if h is None else h.double().cpu().numpy()))
    if bidir:
        out = out + ((None if gf is None else gf.double().cpu().numpy()),)
    return out


def degenerate_inputs(case, Bs=2, L=200, ED=64, seed=13):
    """The scan's special cases: no decay (A = 0: a prefix sum), full decay
    (a underflows to 0: the state restarts every step), steps of zero (a = 1,
    no input), growth (A > 0), no input (x = 0), and all of them mixed."""
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=seed)
    A = inp["A"].copy()
    if case == "no_decay":
        A[:] = 0.0
    elif case == "full_decay":
        A[:] = -1.0e4
    elif case == "growth":
        A[:] = 0.5
    elif case == "zero_steps":
        inp["delta"] = inp["delta"].copy()
        inp["delta"][:, ::2, :] = 0.0
    elif case == "zero_input":
        inp["x"] = np.zeros_like(inp["x"])
    elif case == "mixed":
        A[:, 0:4] = 0.0
        A[:, 4:8] = -1.0e4
        A[:, 8:10] = 0.25
        inp["delta"] = inp["delta"].copy()
        inp["delta"][:, 5::7, :] = 0.0
    inp["A"] = A
    return inp


def options_inputs(Bs, L, ED, dtype, seed):
    """Raw step sizes around softplus^-1 of the usual range, a bias, a gate."""
    inp = synth.make_inputs(Bs, L, ED, 16, "f32", seed=seed)
    raw = (0.7 * synth.normal(seed, 21, (Bs, L, ED)) - 3.5).astype(np.float32)
    z = synth.normal(seed, 22, (Bs, L, ED))
    bias = (0.3 * synth.normal(seed, 23, (ED,))).astype(np.float32)
    inp["delta"] = raw
    if dtype == "bf16":
        for k in ("x", "delta", "B", "C"):
            inp[k] = synth.to_bf16(inp[k])
        z = synth.to_bf16(z)
    return inp, dict(dt_bias=bias, dt_softplus=True, dt_limit=(1e-3, 0.1), z=z)

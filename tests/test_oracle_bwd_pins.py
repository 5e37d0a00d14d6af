"""Pins of the oracle's backward pass (``oracle.scan_bwd``).

The backward pass returns the gradients of L = sum(dy * y) with respect to
every input of the forward scan. It is checked against things other than
itself:
  - central finite differences of the forward oracle (already pinned by
    test_oracle_pins.py), for every input;
  - exact homogeneity identities: y is linear in x and in B when h0 = 0, in C,
    in D x and affine in h0, so <dx, x>, <dB, B>, <dC, C>, <dD, D> and
    <dh0, h0> equal sums of dy times parts of y;
  - the invariance of y under delta -> s delta, A -> A / s, x -> x / s
    (a = exp(delta A) and b = delta x B do not change), whose derivative at
    s = 1 ties ddelta to dA and dx;
  - A = 0, where every gradient has a closed form of prefix sums;
  - reverse-mode differentiation of a plain sequential loop (torch autograd,
    float64, CPU) on tiny inputs.
A slip in the adjoint (a_t for a_{t+1}, h_t for h_{t-1}, a dropped
A a h term in ddelta, a missing D in dx, sums over the wrong axis) fails one
of them.
"""
import numpy as np
import pytest

import oracle
import synth


def inputs(Bs, L, ED, N, seed=0, h0=False):
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=seed)
    # distinct decay per (channel, state) so that a transposed A shows
    inp["A"] = -synth.uniform(seed, 77, (ED, N), 0.5, 4.0)
    inp["delta"] = synth.uniform(seed, 78, (Bs, L, ED), 0.05, 0.6)
    dy = synth.make_output_grad(Bs, L, ED, "f32", seed=seed)
    h = synth.normal(seed, 79, (Bs, ED, N)) if h0 else None
    return inp, dy, h


def loss(inp, dy, h0=None):
    y, _, _ = oracle.scan(**inp, h0=h0)
    return float(np.sum(dy.astype(np.float64) * y))


def fd(inp, dy, h0, name, idx, rel=2.0 ** -9):
    """Central difference of the loss in one float32 input element, with the
    step sizes that float32 actually represents."""
    src = h0 if name == "h0" else inp[name]
    v = float(src[idx])
    s = rel * max(1.0, abs(v))
    up, dn = np.float32(v + s), np.float32(v - s)
    vals = []
    for w in (up, dn):
        arr = src.copy()
        arr[idx] = w
        if name == "h0":
            vals.append(loss(inp, dy, arr))
        else:
            vals.append(loss(dict(inp, **{name: arr}), dy, h0))
    return (vals[0] - vals[1]) / (float(up) - float(dn))


GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "h0"])
def test_backward_matches_finite_differences(name):
    Bs, L, ED, N = 2, 13, 3, 4
    inp, dy, h0 = inputs(Bs, L, ED, N, seed=3, h0=True)
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0)[GRAD_OF[name]]
    shape = h0.shape if name == "h0" else inp[name].shape
    rng = np.random.default_rng(5)
    for _ in range(12):
        idx = tuple(int(rng.integers(0, s)) for s in shape)
        want = fd(inp, dy, h0, name, idx)
        got = g[idx]
        assert abs(got - want) <= 1e-5 * (1.0 + abs(want)), (name, idx, got, want)


@pytest.mark.parametrize("ED", [5, 150])
def test_homogeneity_identities(ED):
    # ED = 150 spans three of the oracle's 64-channel work blocks
    Bs, L, N = 3, 40, 6
    inp, dy, _ = inputs(Bs, L, ED, N, seed=4)
    dy64 = dy.astype(np.float64)
    x64 = inp["x"].astype(np.float64)
    y, _, _ = oracle.scan(**inp)
    dxD = inp["D"].astype(np.float64)[None, None, :] * x64
    g = oracle.scan_bwd(**inp, dy=dy)
    lhs_rhs = [
        (np.sum(g["dx"] * x64), np.sum(dy64 * y)),                  # y linear in x
        (np.sum(g["dB"] * inp["B"]), np.sum(dy64 * (y - dxD))),     # C h linear in B
        (np.sum(g["dC"] * inp["C"]), np.sum(dy64 * (y - dxD))),     # C h linear in C
        (np.sum(g["dD"] * inp["D"]), np.sum(dy64 * dxD)),           # D x
    ]
    for lhs, rhs in lhs_rhs:
        assert abs(lhs - rhs) <= 1e-11 * (1.0 + abs(rhs)), (lhs, rhs)


def test_initial_state_gradient_identity():
    Bs, L, ED, N = 2, 30, 4, 5
    inp, dy, h0 = inputs(Bs, L, ED, N, seed=6, h0=True)
    y1, _, _ = oracle.scan(**inp, h0=h0)
    y0, _, _ = oracle.scan(**inp)
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0)
    lhs = np.sum(g["dh0"] * h0)
    rhs = np.sum(dy.astype(np.float64) * (y1 - y0))
    assert abs(lhs - rhs) <= 1e-11 * (1.0 + abs(rhs))
    # the gradient of h0 does not depend on h0 (y is affine in it)
    g0 = oracle.scan_bwd(**inp, dy=dy, h0=np.zeros_like(h0))
    np.testing.assert_allclose(g["dh0"], g0["dh0"], rtol=0, atol=1e-13)
    # without h0 (the zero initial state) dh0 is the same, and so is dD
    gn = oracle.scan_bwd(**inp, dy=dy)
    np.testing.assert_allclose(gn["dh0"], g["dh0"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gn["dD"], g["dD"], rtol=0, atol=0)


def test_scale_invariance_ties_ddelta_to_dA():
    # y(s delta, A / s, x / s) = y: d/ds at 1 gives <ddelta, delta> - <dA, A> - <dx, x> = 0
    # (the D x term is not invariant: it contributes -<dy, D x>)
    Bs, L, ED, N = 2, 50, 4, 8
    inp, dy, _ = inputs(Bs, L, ED, N, seed=7)
    g = oracle.scan_bwd(**inp, dy=dy)
    x64 = inp["x"].astype(np.float64)
    dxD = np.sum(dy.astype(np.float64) * inp["D"].astype(np.float64)[None, None, :] * x64)
    lhs = np.sum(g["ddelta"] * inp["delta"]) - np.sum(g["dA"] * inp["A"]) - np.sum(g["dx"] * x64)
    assert abs(lhs + dxD) <= 1e-10 * (1.0 + abs(dxD)), (lhs, dxD)


def test_zero_A_closed_form():
    # a = 1: h_t = sum_{s<=t} delta_s x_s B_s, g_t = sum_{s>=t} dy_s C_s
    Bs, L, ED, N = 2, 25, 3, 4
    inp, dy, _ = inputs(Bs, L, ED, N, seed=8)
    inp["A"] = np.zeros((ED, N), np.float32)
    g = oracle.scan_bwd(**inp, dy=dy)
    x = inp["x"].astype(np.float64)
    d = inp["delta"].astype(np.float64)
    B = inp["B"].astype(np.float64)
    C = inp["C"].astype(np.float64)
    dy64 = dy.astype(np.float64)
    D = inp["D"].astype(np.float64)
    u = (d * x)[..., None] * B[:, :, None, :]                 # (Bs, L, ED, N)
    h = np.cumsum(u, axis=1)
    hprev = h - u
    w = dy64[..., None] * C[:, :, None, :]
    gg = np.cumsum(w[:, ::-1], axis=1)[:, ::-1]                # g_t
    np.testing.assert_allclose(g["dC"], np.einsum("ble,blen->bln", dy64, h), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dB"], np.einsum("blen,ble->bln", gg, d * x), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dx"], np.einsum("blen,bln->ble", gg, B) * d + dy64 * D, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["ddelta"], np.einsum("blen,bln->ble", gg, B) * x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dA"], np.einsum("blen,blen,ble->en", gg, hprev, d), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dD"], np.einsum("ble,ble->e", dy64, x), rtol=1e-12, atol=1e-12)


def test_backward_matches_autograd_of_a_plain_loop():
    torch = pytest.importorskip("torch")
    Bs, L, ED, N = 2, 9, 3, 4
    inp, dy, h0 = inputs(Bs, L, ED, N, seed=9, h0=True)
    T = {k: torch.tensor(v.astype(np.float64), requires_grad=True) for k, v in inp.items()}
    th0 = torch.tensor(h0.astype(np.float64), requires_grad=True)
    ys = []
    h = th0
    for t in range(L):
        dt = T["delta"][:, t, :, None]
        h = torch.exp(dt * T["A"][None]) * h + (dt * T["x"][:, t, :, None]) * T["B"][:, t, None, :]
        ys.append((h * T["C"][:, t, None, :]).sum(-1) + T["D"][None] * T["x"][:, t])
    y = torch.stack(ys, 1)
    (y * torch.tensor(dy.astype(np.float64))).sum().backward()
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0)
    for k, name in (("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD")):
        np.testing.assert_allclose(g[name], T[k].grad.numpy(), rtol=1e-12, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(g["dh0"], th0.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_bf16_widens_exactly():
    Bs, L, ED, N = 2, 17, 4, 16
    inp = synth.make_inputs(Bs, L, ED, N, "bf16", seed=2)
    dy = synth.make_output_grad(Bs, L, ED, "bf16", seed=2)
    g16 = oracle.scan_bwd(**inp, dy=dy)
    wide = {k: (synth.from_bf16(v) if v.dtype == np.uint16 else v) for k, v in inp.items()}
    g32 = oracle.scan_bwd(**wide, dy=synth.from_bf16(dy))
    for k in g16:
        np.testing.assert_array_equal(g16[k], g32[k], err_msg=k)


def test_backward_threads_agree():
    Bs, L, ED, N = 5, 33, 6, 16
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=11)
    dy = synth.make_output_grad(Bs, L, ED, "f32", seed=11)
    g1 = oracle.scan_bwd(**inp, dy=dy, nthreads=1)
    g4 = oracle.scan_bwd(**inp, dy=dy, nthreads=4)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g4[k], err_msg=k)


def test_backward_of_empty_inputs():
    # an empty sequence has no output, so every gradient is zero (dh0 too:
    # the loss does not depend on the state); with no channels, dB and dC
    # (sums over the channels) are zero
    inp = synth.make_inputs(2, 0, 6, 16, seed=31)
    h0 = synth.normal(31, 9, (2, 6, 16))
    g = oracle.scan_bwd(**inp, dy=np.zeros((2, 0, 6), np.float32), h0=h0)
    assert g["dx"].shape == (2, 0, 6) and g["dB"].shape == (2, 0, 16)
    for k in ("dA", "dD", "dh0"):
        assert np.array_equal(g[k], np.zeros_like(g[k])), k
    inp = synth.make_inputs(2, 7, 0, 16, seed=32)
    g = oracle.scan_bwd(**inp, dy=np.zeros((2, 7, 0), np.float32))
    assert g["dA"].shape == (0, 16) and g["dD"].shape == (0,)
    for k in ("dB", "dC"):
        assert g[k].shape == (2, 7, 16) and np.array_equal(g[k], np.zeros((2, 7, 16))), k


def bidir_loss(inp, dy, h0=None):
    y, _, _ = oracle.scan(**inp, h0=h0, bidir=True)
    return float(np.sum(dy.astype(np.float64) * y))


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "h0"])
def test_bidirectional_backward_matches_finite_differences(name):
    # central differences of the (pinned) bidirectional forward oracle
    Bs, L, ED, N = 2, 11, 3, 4
    inp, dy, h0 = inputs(Bs, L, ED, N, seed=4, h0=True)
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0, bidir=True)[GRAD_OF[name]]
    shape = h0.shape if name == "h0" else inp[name].shape
    rng = np.random.default_rng(6)
    src = h0 if name == "h0" else inp[name]
    for _ in range(10):
        idx = tuple(int(rng.integers(0, s)) for s in shape)
        v = float(src[idx])
        st = 2.0 ** -11 * max(1.0, abs(v))  # (two directions: more curvature than the forward scan)
        up, dn = np.float32(v + st), np.float32(v - st)
        vals = []
        for w in (up, dn):
            arr = src.copy()
            arr[idx] = w
            vals.append(bidir_loss(inp, dy, arr) if name == "h0" else bidir_loss(dict(inp, **{name: arr}), dy, h0))
        want = (vals[0] - vals[1]) / (float(up) - float(dn))
        assert abs(g[idx] - want) <= 1e-5 * (1.0 + abs(want)), (name, idx, g[idx], want)


def test_bidirectional_backward_identities():
    # y is linear in x (h0 = 0): <dx, x> = <dy, y>; y - D x is linear in C:
    # <dC, C> = <dy, y - D x>; the time flip of every input and of dy maps the
    # bidirectional scan to itself up to which direction carries h0, so with
    # h0 = 0 the gradients flip with the inputs
    inp, dy, _ = inputs(2, 23, 5, 16, seed=8)
    g = oracle.scan_bwd(**inp, dy=dy, bidir=True)
    y, _, _ = oracle.scan(**inp, bidir=True)
    d64 = dy.astype(np.float64)
    assert abs(np.sum(g["dx"] * inp["x"]) - np.sum(d64 * y)) <= 1e-9 * np.sum(np.abs(d64 * y))
    dx_ = inp["D"].astype(np.float64)[None, None, :] * inp["x"]
    assert abs(np.sum(g["dC"] * inp["C"]) - np.sum(d64 * (y - dx_))) <= 1e-9 * np.sum(np.abs(d64 * y))
    flip = lambda a: np.ascontiguousarray(a[:, ::-1])
    fl = {k: (flip(v) if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    gf = oracle.scan_bwd(**fl, dy=flip(dy), bidir=True)
    for k in ("dx", "ddelta", "dB", "dC"):
        assert np.allclose(gf[k][:, ::-1], g[k], rtol=1e-10, atol=1e-12), k
    for k in ("dA", "dD"):
        assert np.allclose(gf[k], g[k], rtol=1e-10, atol=1e-12), k


# ---- the backward through the step-size options and the gate ---------------
OPT_GRAD = dict(GRAD_OF, dt_bias="ddt_bias", z="dz")


def options_case(Bs, L, ED, N, seed):
    inp, dy, h0 = inputs(Bs, L, ED, N, seed=seed, h0=True)
    inp["delta"] = synth.uniform(seed, 80, (Bs, L, ED), -3.0, 1.0)   # raw step sizes (softplus makes them > 0)
    opts = dict(dt_bias=(0.5 * synth.normal(seed, 81, (ED,)) - 0.5).astype(np.float32), dt_softplus=True,
                dt_limit=(0.08, 0.6), z=synth.normal(seed, 82, (Bs, L, ED)))
    return inp, dy, h0, opts


def options_loss(inp, dy, h0, opts, bidir):
    y, _, _ = oracle.scan(**inp, h0=h0, bidir=bidir, **opts)
    return float(np.sum(dy.astype(np.float64) * y))


@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "h0", "dt_bias", "z"])
def test_options_backward_matches_finite_differences(name, bidir):
    # central differences of the (pinned) forward oracle with bias, softplus,
    # a clamp that binds on some steps, and the gate
    Bs, L, ED, N = 2, 11, 3, 4
    inp, dy, h0, opts = options_case(Bs, L, ED, N, seed=5)
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0, bidir=bidir, **opts)[OPT_GRAD[name]]
    src = h0 if name == "h0" else (opts[name] if name in ("dt_bias", "z") else inp[name])
    rng = np.random.default_rng(7)
    lo, hi = opts["dt_limit"]
    checked = 0
    for _ in range(14):
        idx = tuple(int(rng.integers(0, s)) for s in src.shape)
        v = float(src[idx])
        st = 2.0 ** -11 * max(1.0, abs(v))
        if name in ("delta", "dt_bias"):
            # skip points whose mapped step size lies within a few steps of a
            # clamp bound (the map has a kink there)
            e = idx[-1]
            raw = inp["delta"][..., e] + opts["dt_bias"][e]
            u = np.where(raw > 20, raw, np.log1p(np.exp(raw.astype(np.float64))))
            near = np.abs(u - lo) < 8 * st if name == "dt_bias" else abs(u[idx[:-1]] - lo) < 8 * st
            near = np.any(near) or np.any(np.abs(u - hi) < 8 * st) if name == "dt_bias" else \
                near or abs(u[idx[:-1]] - hi) < 8 * st
            if near:
                continue
        up, dn = np.float32(v + st), np.float32(v - st)
        vals = []
        for w in (up, dn):
            arr = src.copy()
            arr[idx] = w
            if name == "h0":
                vals.append(options_loss(inp, dy, arr, opts, bidir))
            elif name in ("dt_bias", "z"):
                vals.append(options_loss(inp, dy, h0, dict(opts, **{name: arr}), bidir))
            else:
                vals.append(options_loss(dict(inp, **{name: arr}), dy, h0, opts, bidir))
        want = (vals[0] - vals[1]) / (float(up) - float(dn))
        assert abs(g[idx] - want) <= 1e-5 * (1.0 + abs(want)), (name, bidir, idx, g[idx], want)
        checked += 1
    assert checked >= 5


def test_options_backward_clamped_steps_have_no_gradient():
    # a step size held at a clamp bound does not move with its raw value
    inp, dy, h0, opts = options_case(2, 40, 5, 16, seed=9)
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0, **opts)
    raw = inp["delta"].astype(np.float64) + opts["dt_bias"][None, None, :]
    u = np.log1p(np.exp(raw))
    clamped = (u <= opts["dt_limit"][0]) | (u >= opts["dt_limit"][1])
    assert clamped.any() and (~clamped).any()
    assert np.all(g["ddelta"][clamped] == 0.0)
    assert np.all(g["ddelta"][~clamped] != 0.0)
    # ddt_bias is the sum of the raw step sizes' gradients over batch rows and time
    np.testing.assert_allclose(g["ddt_bias"], g["ddelta"].sum(axis=(0, 1)), rtol=1e-12, atol=1e-14)


def test_no_options_equals_plain_backward():
    inp, dy, h0 = inputs(2, 30, 4, 16, seed=10, h0=True)
    a = oracle.scan_bwd(**inp, dy=dy, h0=h0)
    b = oracle.scan_bwd(**inp, dy=dy, h0=h0, dt_bias=np.zeros(4, np.float32))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    np.testing.assert_allclose(b["ddt_bias"], a["ddelta"].sum(axis=(0, 1)), rtol=1e-12, atol=1e-14)

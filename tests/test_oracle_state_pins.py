"""Pins of the oracle's carried states in both directions.

The Bi-Mamba2 forward returns a final state per direction (final_states_f,
final_states_b), and its backward takes their gradient (dfinal_states):
"Some questions of Bi-Mamba2 and Hydra", the MambaChunkScanCombinedFn
listings. So the oracle takes, besides h0, a reverse state g0 entering the
bidirectional scan's reverse direction at the last step, and its backward
takes dh_last (and, bidirectional, dg_first) and returns dg0 beside dh0.

Each of these is checked against something other than the oracle's own
arithmetic for it:
  - g0: a bidirectional sequence cut in two pieces composes back to the
    whole (the reverse state flows from the later piece into the earlier
    one, the forward state the other way), bit for bit; the g0-only part of
    y equals its closed form sum_n C_t[n] (prod_{s >= t} a_s[n]) g0[n]
    written with numpy cumulative products; and the flip identity with the
    (already pinned) forward scan started from h0 = g0;
  - dh_last, dg_first, dg0: central finite differences of the forward oracle
    for L = sum(dy y) + sum(dh_last h_last) + sum(dg_first g_first); closed
    forms for dy = 0 (dh0 = prod(a) dh_last, dx_t = delta_t sum_n (prod_{s>t}
    a_s) dh_last B_t); and the homogeneity <dx, x> = <dy, y> +
    <dh_last, h_last> (y and h_last are linear in x for h0 = 0).
Planted slips (g0 ignored, g0 entering at t = 0, dh_last added after the
last step's decay, dg_first sent to the forward adjoint) each fail one.
"""
import numpy as np
import pytest

import oracle
import synth


def inputs(Bs, L, ED, N, seed):
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=seed)
    inp["A"] = -synth.uniform(seed, 77, (ED, N), 0.5, 4.0)
    inp["delta"] = synth.uniform(seed, 78, (Bs, L, ED), 0.05, 0.6)
    return inp


def states(seed, stream, Bs, ED, N):
    return synth.normal(seed, stream, (Bs, ED, N))


def piece(inp, lo, hi):
    return {k: (np.ascontiguousarray(v[:, lo:hi]) if v.ndim == 3 else v) for k, v in inp.items()}


def decays(inp):
    """a_t[b, t, e, n] = exp(delta A) in fp64"""
    d = inp["delta"].astype(np.float64)[..., None]
    return np.exp(d * inp["A"].astype(np.float64)[None, None])


# --- g0: the reverse direction's initial state ---------------------------------
@pytest.mark.parametrize("L1", [1, 7, 20, 39])
def test_bidirectional_two_pieces_compose(L1):
    Bs, L, ED, N = 2, 40, 5, 6
    inp = inputs(Bs, L, ED, N, seed=11)
    H, G = states(11, 90, Bs, ED, N), states(11, 91, Bs, ED, N)
    y, hl, gf = oracle.scan(**inp, h0=H, g0=G, bidir=True, want_h_last=True, want_g_first=True)
    p1, p2 = piece(inp, 0, L1), piece(inp, L1, L)
    # the reverse state of the later piece does not depend on the forward one
    _, _, g2 = oracle.scan(**p2, g0=G, bidir=True, want_g_first=True)
    y1, h1, g1 = oracle.scan(**p1, h0=H, g0=g2.astype(np.float32), bidir=True, want_h_last=True,
                             want_g_first=True)
    y2, h2, _ = oracle.scan(**p2, h0=h1.astype(np.float32), g0=G, bidir=True, want_h_last=True)
    # states cross the cut as float32 (as a caller's buffers carry them): equal to rounding
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(h2, hl, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(g1, gf, rtol=1e-6, atol=1e-6)


def test_bidirectional_two_pieces_compose_exactly_with_exact_states():
    # with states that are exact in float32 (the pieces' own results rounded
    # back into the full run) the composition is bit for bit
    Bs, L, ED, N, L1 = 1, 24, 3, 4, 10
    inp = inputs(Bs, L, ED, N, seed=12)
    p1, p2 = piece(inp, 0, L1), piece(inp, L1, L)
    _, _, g2 = oracle.scan(**p2, bidir=True, want_g_first=True)
    _, h1, _ = oracle.scan(**p1, want_h_last=True)
    g2f, h1f = g2.astype(np.float32), h1.astype(np.float32)
    ya, _, _ = oracle.scan(**p1, g0=g2f, bidir=True)
    yb, _, _ = oracle.scan(**p2, h0=h1f, bidir=True)
    # reference: each piece's missing direction entered from the same float32 state
    y1r, _, _ = oracle.scan(**p1, bidir=True)
    y2r, _, _ = oracle.scan(**p2, bidir=True)
    a = decays(inp)
    C = inp["C"].astype(np.float64)
    # contributions of the carried states, closed form
    Pr = np.flip(np.cumprod(np.flip(a[:, :L1], 1), axis=1), 1)         # prod_{s=t..L1-1} a_s
    Pf = np.cumprod(a[:, L1:], axis=1)                                  # prod_{s=L1..t} a_s
    add1 = np.einsum("btn,bten,ben->bte", C[:, :L1], Pr, g2f.astype(np.float64))
    add2 = np.einsum("btn,bten,ben->bte", C[:, L1:], Pf, h1f.astype(np.float64))
    np.testing.assert_allclose(ya, y1r + add1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(yb, y2r + add2, rtol=1e-12, atol=1e-12)


def test_g0_part_closed_form_and_flip_identity():
    Bs, L, ED, N = 2, 17, 4, 5
    inp = inputs(Bs, L, ED, N, seed=13)
    G = states(13, 92, Bs, ED, N)
    y1, _, g1 = oracle.scan(**inp, g0=G, bidir=True, want_g_first=True)
    y0, _, g0r = oracle.scan(**inp, bidir=True, want_g_first=True)
    a = decays(inp)
    P = np.flip(np.cumprod(np.flip(a, 1), axis=1), 1)                   # prod_{s >= t} a_s
    want = np.einsum("btn,bten,ben->bte", inp["C"].astype(np.float64), P, G.astype(np.float64))
    np.testing.assert_allclose(y1 - y0, want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g1 - g0r, P[:, 0] * G, rtol=1e-11, atol=1e-12)
    # flip identity: the reverse direction is the forward scan of the flipped
    # inputs started from h0 = g0 (no D), flipped back
    flip = lambda v: np.ascontiguousarray(v[:, ::-1])
    yf, _, _ = oracle.scan(**inp)
    fl = {k: (flip(v) if v.ndim == 3 else v) for k, v in inp.items()}
    yr, hr, _ = oracle.scan(**dict(fl, D=None), h0=G, want_h_last=True)
    np.testing.assert_allclose(y1, yf + yr[:, ::-1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1, hr, rtol=0, atol=0)


# --- gradients of the carried states ---------------------------------------------
def total_loss(inp, dy, h0, g0, dhl, dgf, bidir):
    y, hl, gf = oracle.scan(**inp, h0=h0, g0=g0, bidir=bidir, want_h_last=True, want_g_first=bidir)
    L = np.sum(dy.astype(np.float64) * y) + np.sum(dhl.astype(np.float64) * hl)
    if bidir:
        L += np.sum(dgf.astype(np.float64) * gf)
    return float(L)


def fd(inp, dy, h0, g0, dhl, dgf, bidir, name, idx, rel=2.0 ** -9):
    src = {"h0": h0, "g0": g0}.get(name, inp.get(name))
    v = float(src[idx])
    s = rel * max(1.0, abs(v))
    up, dn = np.float32(v + s), np.float32(v - s)
    vals = []
    for w in (up, dn):
        arr = src.copy()
        arr[idx] = w
        kw = dict(h0=h0, g0=g0)
        if name in kw:
            kw[name] = arr
            vals.append(total_loss(inp, dy, kw["h0"], kw["g0"], dhl, dgf, bidir))
        else:
            vals.append(total_loss(dict(inp, **{name: arr}), dy, h0, g0, dhl, dgf, bidir))
    return (vals[0] - vals[1]) / (float(up) - float(dn))


GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0", "g0": "dg0"}


@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "h0", "g0"])
def test_state_gradients_match_finite_differences(name, bidir):
    if name == "g0" and not bidir:
        pytest.skip("g0 belongs to the bidirectional scan")
    Bs, L, ED, N = 2, 11, 3, 4
    inp = inputs(Bs, L, ED, N, seed=14)
    dy = synth.make_output_grad(Bs, L, ED, "f32", seed=14)
    h0, g0 = states(14, 93, Bs, ED, N), (states(14, 94, Bs, ED, N) if bidir else None)
    dhl = states(14, 95, Bs, ED, N)
    dgf = states(14, 96, Bs, ED, N) if bidir else None
    g = oracle.scan_bwd(**inp, dy=dy, h0=h0, g0=g0, dh_last=dhl, dg_first=dgf, bidir=bidir)[GRAD_OF[name]]
    src = {"h0": h0, "g0": g0}.get(name, inp.get(name))
    rng = np.random.default_rng(6)
    for _ in range(10):
        idx = tuple(int(rng.integers(0, s)) for s in src.shape)
        want = fd(inp, dy, h0, g0, dhl, dgf, bidir, name, idx)
        assert abs(g[idx] - want) <= 1e-5 * (1.0 + abs(want)), (name, idx, g[idx], want)


def test_final_state_gradient_closed_forms():
    # dy = 0: only the final state is in the loss
    Bs, L, ED, N = 2, 15, 3, 5
    inp = inputs(Bs, L, ED, N, seed=15)
    dhl = states(15, 97, Bs, ED, N)
    dy = np.zeros((Bs, L, ED), np.float32)
    g = oracle.scan_bwd(**inp, dy=dy, dh_last=dhl)
    a = decays(inp)
    total = np.prod(a, axis=1)                                          # prod over all t
    np.testing.assert_allclose(g["dh0"], total * dhl, rtol=1e-12, atol=1e-14)
    # prod_{s > t} a_s, shifted so that the last step has the empty product 1
    after = np.concatenate([np.flip(np.cumprod(np.flip(a[:, 1:], 1), axis=1), 1),
                            np.ones_like(a[:, :1])], axis=1)
    B64, d64 = inp["B"].astype(np.float64), inp["delta"].astype(np.float64)
    want_dx = d64 * np.einsum("bten,ben,btn->bte", after, dhl.astype(np.float64), B64)
    np.testing.assert_allclose(g["dx"], want_dx, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dC"], 0.0, atol=0)
    np.testing.assert_allclose(g["dD"], 0.0, atol=0)


def test_final_state_homogeneity():
    Bs, L, ED, N = 3, 30, 70, 4  # 70 channels: two of the oracle's channel blocks
    inp = inputs(Bs, L, ED, N, seed=16)
    dy = synth.make_output_grad(Bs, L, ED, "f32", seed=16)
    dhl = states(16, 98, Bs, ED, N)
    y, hl, _ = oracle.scan(**inp, want_h_last=True)
    g = oracle.scan_bwd(**inp, dy=dy, dh_last=dhl)
    lhs = np.sum(g["dx"] * inp["x"].astype(np.float64))
    rhs = np.sum(dy.astype(np.float64) * y) + np.sum(dhl.astype(np.float64) * hl)
    assert abs(lhs - rhs) <= 1e-11 * (1.0 + abs(rhs))
    # and B: sum(dB B) = <dy, y - D x> + <dh_last, h_last>
    dxD = inp["D"].astype(np.float64)[None, None, :] * inp["x"].astype(np.float64)
    lhs = np.sum(g["dB"] * inp["B"].astype(np.float64))
    rhs = np.sum(dy.astype(np.float64) * (y - dxD)) + np.sum(dhl.astype(np.float64) * hl)
    assert abs(lhs - rhs) <= 1e-11 * (1.0 + abs(rhs))


def test_reverse_state_gradient_mirrors_forward():
    # the bidirectional backward with dy = 0 and only dg_first is the forward
    # backward of the flipped inputs with dh_last = dg_first, flipped back
    Bs, L, ED, N = 2, 12, 3, 4
    inp = inputs(Bs, L, ED, N, seed=17)
    dgf = states(17, 99, Bs, ED, N)
    zero = np.zeros((Bs, L, ED), np.float32)
    g = oracle.scan_bwd(**inp, dy=zero, dg_first=dgf, bidir=True)
    a = decays(inp)
    np.testing.assert_allclose(g["dg0"], np.prod(a, axis=1) * dgf, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dh0"], 0.0, atol=0)
    # dx_t = delta_t sum_n (prod_{s < t} a_s) dg_first B_t
    before = np.concatenate([np.ones_like(a[:, :1]), np.cumprod(a[:, :-1], axis=1)], axis=1)
    want = inp["delta"].astype(np.float64) * np.einsum("bten,ben,btn->bte", before, dgf.astype(np.float64),
                                                       inp["B"].astype(np.float64))
    np.testing.assert_allclose(g["dx"], want, rtol=1e-12, atol=1e-14)


def test_ssd_reverse_initial_state():
    # the multi-head form with g0 equals the per-channel oracle with g0 expanded
    Bs, L, H, P, G, N = 2, 9, 4, 3, 2, 5
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, "f32", seed=18)
    g0 = synth.normal(18, 100, (Bs, H, P, N))
    y, _, gf = oracle.ssd(**inp, g0=g0, bidir=True, want_g_first=True)
    # expand: channel e = h * P + p, A[e, n] = A[h], delta[e] = dt[h], B, C of the head's group
    ED = H * P
    heads = np.arange(ED) // P
    grp = heads // (H // G)
    for gi in range(G):
        sel = np.nonzero(grp == gi)[0]
        x = np.ascontiguousarray(inp["x"].reshape(Bs, L, ED)[:, :, sel])
        dl = np.ascontiguousarray(inp["dt"][:, :, heads[sel]])
        A = np.ascontiguousarray(np.repeat(inp["A"][heads[sel]][:, None], N, axis=1))
        Bg = np.ascontiguousarray(inp["B"][:, :, gi])
        Cg = np.ascontiguousarray(inp["C"][:, :, gi])
        D = np.ascontiguousarray(inp["D"][heads[sel]])
        g0e = np.ascontiguousarray(g0.reshape(Bs, ED, N)[:, sel])
        ye, _, ge = oracle.scan(x, dl, A, Bg, Cg, D, g0=g0e, bidir=True, want_g_first=True)
        np.testing.assert_allclose(y.reshape(Bs, L, ED)[:, :, sel], ye, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gf.reshape(Bs, ED, N)[:, sel], ge, rtol=1e-12, atol=1e-12)

"""Pins of the multi-head (SSD) oracle (``oracle.ssd``).

It is checked against things other than itself: the already pinned
per-channel oracle (``oracle.scan``) on the same inputs expanded to one
channel per (head, head channel), group by group; the closed (semiseparable
matrix) form written out with its decay products; the bidirectional sum as
forward plus flipped forward; the split / resume composition of the final
state; bf16 widening; and thread-count invariance. A slip (the wrong group's
B, a per-state instead of per-head decay, C applied before the update, a
reverse scan with a_{t+1}) fails one of them.
"""
import numpy as np
import pytest

import oracle
import synth


def rel(a, b):
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b))))


@pytest.mark.parametrize("G", [1, 2])
def test_equals_per_channel_scan_group_by_group(G):
    Bs, L, H, P, N = 2, 37, 4, 3, 5
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, seed=1)
    h0 = synth.normal(1, 90, (Bs, H, P, N))
    y, hl, _ = oracle.ssd(**inp, h0=h0, want_h_last=True)
    hpg = H // G
    for g in range(G):
        heads = list(range(g * hpg, (g + 1) * hpg))
        ED = hpg * P
        x = np.ascontiguousarray(inp["x"][:, :, heads, :].reshape(Bs, L, ED))
        delta = np.ascontiguousarray(np.repeat(inp["dt"][:, :, heads], P, axis=2))
        A = np.ascontiguousarray(np.repeat(inp["A"][heads], P)[:, None] * np.ones((1, N), np.float32))
        D = np.ascontiguousarray(np.repeat(inp["D"][heads], P))
        B = np.ascontiguousarray(inp["B"][:, :, g, :])
        C = np.ascontiguousarray(inp["C"][:, :, g, :])
        h0e = np.ascontiguousarray(h0[:, heads].reshape(Bs, ED, N))
        y1, h1, _ = oracle.scan(x, delta, A, B, C, D, h0=h0e, want_h_last=True)
        np.testing.assert_array_equal(y[:, :, heads, :].reshape(Bs, L, ED), y1)
        np.testing.assert_array_equal(hl[:, heads].reshape(Bs, ED, N), h1)


@pytest.mark.parametrize("G,bidir", [(1, False), (2, False), (2, True)])
def test_options_equal_per_channel_options(G, bidir):
    # dt_bias per head, softplus, a clamp that binds at both ends, and the
    # gate, against the per-channel oracle's (separately pinned) options on
    # the expanded inputs
    Bs, L, H, P, N = 2, 29, 4, 3, 5
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, seed=11)
    inp["dt"] = synth.normal(11, 95, (Bs, L, H))           # raw, both signs
    dt_bias = synth.normal(11, 96, (H,))
    z = synth.normal(11, 97, (Bs, L, H, P))
    h0 = synth.normal(11, 98, (Bs, H, P, N))
    opts = dict(dt_bias=dt_bias, dt_softplus=True, dt_limit=(0.05, 1.2), z=z)
    y, hl, gf = oracle.ssd(**inp, h0=h0, bidir=bidir, want_h_last=True, want_g_first=bidir, **opts)
    y0, _, _ = oracle.ssd(**inp, h0=h0, bidir=bidir)
    assert rel(y, y0) > 1e-2                                # the options change the result
    hpg = H // G
    for g in range(G):
        heads = list(range(g * hpg, (g + 1) * hpg))
        ED = hpg * P
        x = np.ascontiguousarray(inp["x"][:, :, heads, :].reshape(Bs, L, ED))
        delta = np.ascontiguousarray(np.repeat(inp["dt"][:, :, heads], P, axis=2))
        A = np.ascontiguousarray(np.repeat(inp["A"][heads], P)[:, None] * np.ones((1, N), np.float32))
        D = np.ascontiguousarray(np.repeat(inp["D"][heads], P))
        B = np.ascontiguousarray(inp["B"][:, :, g, :])
        C = np.ascontiguousarray(inp["C"][:, :, g, :])
        h0e = np.ascontiguousarray(h0[:, heads].reshape(Bs, ED, N))
        ze = np.ascontiguousarray(z[:, :, heads, :].reshape(Bs, L, ED))
        be = np.ascontiguousarray(np.repeat(dt_bias[heads], P))
        y1, h1, g1 = oracle.scan(x, delta, A, B, C, D, h0=h0e, dt_bias=be, dt_softplus=True, dt_limit=(0.05, 1.2),
                                 z=ze, bidir=bidir, want_h_last=True, want_g_first=bidir)
        # the bidirectional sums add the D x term in another order
        assert rel(y[:, :, heads, :].reshape(Bs, L, ED), y1) < 1e-13
        assert rel(hl[:, heads].reshape(Bs, ED, N), h1) == 0.0
        if bidir:
            assert rel(gf[:, heads].reshape(Bs, ED, N), g1) == 0.0


def test_closed_matrix_form():
    # y_t = sum_{s <= t} (C_t . B_s) exp(A sum_{r=s+1}^{t} dt_r) dt_s x_s + D x_t
    #       + sum_n C_t[n] exp(A sum_{r<=t} dt_r) h0[n]
    Bs, L, H, P, G, N = 1, 23, 2, 3, 1, 4
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, seed=2)
    h0 = synth.normal(2, 91, (Bs, H, P, N))
    y, _, _ = oracle.ssd(**inp, h0=h0)
    x = inp["x"].astype(np.float64)[0]
    dt = inp["dt"].astype(np.float64)[0]
    B = inp["B"].astype(np.float64)[0, :, 0]
    C = inp["C"].astype(np.float64)[0, :, 0]
    ref = np.zeros((L, H, P))
    for h in range(H):
        A = float(inp["A"][h])
        for t in range(L):
            for s in range(t + 1):
                decay = np.exp(A * dt[s + 1:t + 1, h].sum())
                ref[t, h] += (C[t] @ B[s]) * decay * dt[s, h] * x[s, h]
            ref[t, h] += np.exp(A * dt[:t + 1, h].sum()) * (h0[0, h].astype(np.float64) @ C[t])
            ref[t, h] += inp["D"][h] * x[t, h]
    assert rel(y[0], ref) < 1e-12


def test_bidirectional_is_forward_plus_flipped_forward():
    Bs, L, H, P, G, N = 2, 19, 4, 2, 2, 3
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, seed=3)
    yb, _, gf = oracle.ssd(**inp, bidir=True, want_g_first=True)
    yf, _, _ = oracle.ssd(**inp)
    flip = {k: (np.ascontiguousarray(v[:, ::-1]) if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    yr, hr, _ = oracle.ssd(**dict(flip, D=None), want_h_last=True)
    assert rel(yb, yf + yr[:, ::-1]) < 1e-13
    assert rel(gf, hr) < 1e-13


def test_final_state_resumes():
    Bs, L, H, P, G, N = 2, 40, 2, 3, 1, 4
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, seed=4)
    L1 = 17
    pre = {k: (np.ascontiguousarray(v[:, :L1]) if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    suf = {k: (np.ascontiguousarray(v[:, L1:]) if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y, hl, _ = oracle.ssd(**inp, want_h_last=True)
    _, h1, _ = oracle.ssd(**pre, want_h_last=True)
    # exact resume needs the float64 carried state: compare through float32 rounding
    y2, h2, _ = oracle.ssd(**suf, h0=h1.astype(np.float32), want_h_last=True)
    assert rel(y2, y[:, L1:]) < 1e-6 and rel(h2, hl) < 1e-6


def test_zero_dt_is_constant_state_and_skip_term():
    Bs, L, H, P, G, N = 1, 9, 2, 2, 1, 3
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, seed=5)
    inp["dt"] = np.zeros_like(inp["dt"])
    h0 = synth.normal(5, 92, (Bs, H, P, N))
    y, hl, _ = oracle.ssd(**inp, h0=h0, want_h_last=True)
    # a = 1, no input: the state stays h0 and y_t = C_t h0 + D x_t
    np.testing.assert_array_equal(hl, h0.astype(np.float64))
    ref = np.einsum("ltn,hpn->lthp", inp["C"][0].astype(np.float64)[:, None, 0, :].repeat(1, 1),
                    h0[0].astype(np.float64))[:, 0] + inp["D"][None, :, None] * inp["x"][0].astype(np.float64)
    assert rel(y[0], ref) < 1e-14


def test_bf16_widens_exactly_and_threads_agree():
    Bs, L, H, P, G, N = 3, 21, 4, 8, 1, 16
    inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, "bf16", seed=6)
    y16, _, _ = oracle.ssd(**inp, nthreads=1)
    wide = {k: (synth.from_bf16(v) if v.dtype == np.uint16 else v) for k, v in inp.items()}
    y32, _, _ = oracle.ssd(**wide, nthreads=5)
    np.testing.assert_array_equal(y16, y32)


def test_empty_sequence_keeps_the_entering_state():
    Bs, H, P, G, N = 2, 4, 3, 2, 5
    inp = synth.make_ssd_inputs(Bs, 0, H, P, G, N, seed=8)
    h0 = synth.normal(8, 9, (Bs, H, P, N))
    y, hl, gf = oracle.ssd(**inp, h0=h0, bidir=True, want_h_last=True, want_g_first=True)
    assert y.shape == (Bs, 0, H, P)
    assert np.array_equal(hl, h0.astype(np.float64)) and np.array_equal(gf, np.zeros((Bs, H, P, N)))
    y0, _, _ = oracle.ssd(**synth.make_ssd_inputs(0, 6, H, P, G, N, seed=8))
    assert y0.shape == (0, 6, H, P)


def test_rejects_bad_arguments():
    inp = synth.make_ssd_inputs(1, 4, 3, 2, 1, 2, seed=7)
    with pytest.raises(RuntimeError):
        oracle.ssd(**dict(inp, B=np.zeros((1, 4, 2, 2), np.float32), C=np.zeros((1, 4, 2, 2), np.float32)))

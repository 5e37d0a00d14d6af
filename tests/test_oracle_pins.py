"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle (``oracle.scan``) against something other than
itself: the pages' worked example of the parallel scan, closed forms, special
cases that reduce to a library routine, brute force on tiny inputs and the
agreement of sequential / parallel / chunkwise forms. A plausible slip in the
oracle (a dropped D term, a wrong sign in the exponent, B_{t-1} for B_t, a
transposed A, a reverse scan that uses a_{t+1}) fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# A parallel (tree) scan written from the definition of an inclusive scan with
# an associative operator: combine neighbouring elements in pairs, scan the
# half-length sequence of pair results recursively, then each odd position
# takes its pair's scanned value and each even position (but the first)
# combines the previous pair's scanned value with its own element. This is
# the pairwise reduction followed by the fill-in that the page "scan output is
# different between sequential and parallel versions" describes (its issue
# text and the author's reply), organised as a recursion; its worked example
# pins the 1-D (additive) case below. Power-of-two lengths only, as there.
# ---------------------------------------------------------------------------
def tree_scan(xs, combine):
    """Inclusive scan of the list xs under an associative combine(earlier, later)."""
    n = len(xs)
    if n == 1:
        return list(xs)
    assert n % 2 == 0, "power-of-two lengths only"
    pairs = [combine(xs[2 * i], xs[2 * i + 1]) for i in range(n // 2)]
    scanned = tree_scan(pairs, combine)
    out = [None] * n
    out[0] = xs[0]
    for i in range(n // 2):
        out[2 * i + 1] = scanned[i]
        if i > 0:
            out[2 * i] = combine(scanned[i - 1], xs[2 * i])
    return out


def sweep_1d(values):
    """The tree scan with addition: exact on integers."""
    return np.array(tree_scan([int(v) for v in values], lambda u, v: u + v), dtype=np.int64)


def sweep_pairs(a, b):
    """The tree scan of the pair operator (a1, b1) then (a2, b2) -> (a1 a2,
    a2 b1 + b2): each pair is the affine map h -> a h + b, and the scan of
    the maps gives h_t with h_{-1} = 0.

    a, b: arrays with time on axis 0 (power-of-two length). Returns h (the
    b part of the inclusive scan), in a's and b's dtype.
    """
    a = np.asarray(a)
    b = np.asarray(b)
    combine = lambda e1, e2: (e1[0] * e2[0], e2[0] * e1[1] + e2[1])
    scanned = tree_scan([(a[t], b[t]) for t in range(a.shape[0])], combine)
    return np.stack([s[1] for s in scanned]).astype(np.result_type(a, b), copy=False)


def discretise(x, delta, A, B):
    """(a, b) pairs with time on axis 0: a (L, Bs, ED, N), b (L, Bs, ED, N)."""
    d = delta.astype(np.float64).transpose(1, 0, 2)[..., None]        # (L, Bs, ED, 1)
    xv = x.astype(np.float64).transpose(1, 0, 2)[..., None]
    a = np.exp(d * A.astype(np.float64)[None, None, :, :])            # (L, Bs, ED, N)
    b = (d * xv) * B.astype(np.float64).transpose(1, 0, 2)[:, :, None, :]
    return a, b


def contract(h, C, x, D):
    """y (Bs, L, ED) from states h (L, Bs, ED, N)."""
    Ct = C.astype(np.float64).transpose(1, 0, 2)[:, :, None, :]        # (L, Bs, 1, N)
    y = (h * Ct).sum(-1).transpose(1, 0, 2)
    if D is not None:
        y = y + D.astype(np.float64)[None, None, :] * x.astype(np.float64)
    return y


def small_inputs(Bs, L, ED, N, seed=0, distinct_A=True):
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=seed)
    if distinct_A:
        # per-channel, per-state decay rates so that a transposed A shows
        inp["A"] = -synth.uniform(seed, 77, (ED, N), 0.5, 4.0)
    return inp


def rel_err(a, b):
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b))))


# --- Pin 1: the pages' worked example -------------------------------------
def test_pages_worked_example_1d_sweep():
    with open(os.path.join(HERE, "golden", "pscan_1d_example.txt")) as f:
        rows = [l.split(":") for l in f if not l.startswith("#") and ":" in l]
    fixture = {k.strip(): [int(v) for v in vals.split()] for k, vals in rows}
    out = sweep_1d(fixture["input"])
    assert out.tolist() == fixture["output"]
    assert out.tolist() == np.cumsum(fixture["input"]).tolist()


def test_pair_sweep_reduces_to_1d_sweep():
    vals = np.arange(1, 17, dtype=np.float64)
    h = sweep_pairs(np.ones(16), vals)
    assert h.tolist() == sweep_1d(np.arange(1, 17)).tolist()


# --- Pin 4 / 7: sequential (oracle) == parallel (pages' sweep) ---------------
@pytest.mark.parametrize("L", [1, 2, 8, 64, 256])
def test_oracle_equals_parallel_sweep(L):
    inp = small_inputs(2, L, 6, 5, seed=L)
    y, h_last, _ = oracle.scan(**inp, want_h_last=True)
    a, b = discretise(inp["x"], inp["delta"], inp["A"], inp["B"])
    h = sweep_pairs(a, b)
    y_ref = contract(h, inp["C"], inp["x"], inp["D"])
    assert rel_err(y, y_ref) < 1e-12
    assert rel_err(h_last, h[-1]) < 1e-12


def test_pages_recipe_seq_vs_parallel_fp32():
    # the pages' own check: Bs=2, L=64, D=32 (ED = 2D = 64), N=16, every input
    # standard normal (A and delta too), parallel vs sequential, rtol 0.01,
    # here with the parallel side in float32.
    Bs, L, ED, N = 2, 64, 64, 16
    g = lambda s, shape: synth.normal(1234, s, shape)
    x, delta, A = g(1, (Bs, L, ED)), g(2, (Bs, L, ED)), g(3, (ED, N))
    B, C, D = g(4, (Bs, L, N)), g(5, (Bs, L, N)), g(6, (ED,))
    y, _, _ = oracle.scan(x, delta, A, B, C, D)
    a, b = discretise(x, delta, A, B)
    h32 = sweep_pairs(a.astype(np.float32), b.astype(np.float32))
    y32 = contract(h32, C, x, D)
    assert np.allclose(y32, y, rtol=0.01)


# --- Pin 3: brute-force closed form on tiny inputs --------------------------
def test_oracle_equals_closed_form_sum():
    Bs, L, ED, N = 2, 11, 3, 4
    inp = small_inputs(Bs, L, ED, N, seed=3)
    y, h_last, _ = oracle.scan(**inp, want_h_last=True)
    a, b = discretise(inp["x"], inp["delta"], inp["A"], inp["B"])
    h = np.zeros_like(b)
    for t in range(L):
        for s in range(t + 1):
            w = np.ones_like(a[0])
            for r in range(s + 1, t + 1):
                w = w * a[r]
            h[t] += w * b[s]
    assert rel_err(y, contract(h, inp["C"], inp["x"], inp["D"])) < 1e-13
    assert rel_err(h_last, h[-1]) < 1e-13


# --- Pin 4: chunkwise form with carries --------------------------------------
@pytest.mark.parametrize("chunk", [1, 3, 4, 7, 40])
def test_oracle_equals_chunkwise_form(chunk):
    Bs, L, ED, N = 2, 40, 4, 6
    inp = small_inputs(Bs, L, ED, N, seed=chunk)
    y, _, _ = oracle.scan(**inp)
    a, b = discretise(inp["x"], inp["delta"], inp["A"], inp["B"])
    h = np.zeros_like(b)
    carry = np.zeros_like(b[0])
    for s0 in range(0, L, chunk):
        s1 = min(L, s0 + chunk)
        P = np.cumprod(a[s0:s1], axis=0)                 # prod of a over [s0, t]
        local = np.zeros_like(b[s0:s1])                  # scan of the chunk from zero
        acc = np.zeros_like(b[0])
        for t in range(s1 - s0):
            acc = a[s0 + t] * acc + b[s0 + t]
            local[t] = acc
        h[s0:s1] = local + P * carry[None]
        carry = h[s1 - 1]
    assert rel_err(y, contract(h, inp["C"], inp["x"], inp["D"])) < 1e-12


# --- Pin 2: A = 0 reduces the scan to a prefix sum ----------------------------
def test_zero_A_is_prefix_sum_exact():
    Bs, L, ED, N = 2, 50, 5, 4
    rng = np.random.default_rng(0)
    x = rng.integers(-3, 4, (Bs, L, ED)).astype(np.float32)
    delta = np.ones((Bs, L, ED), np.float32)
    B = rng.integers(-2, 3, (Bs, L, N)).astype(np.float32)
    C = rng.integers(-2, 3, (Bs, L, N)).astype(np.float32)
    D = rng.integers(-2, 3, (ED,)).astype(np.float32)
    A = np.zeros((ED, N), np.float32)
    y, h_last, _ = oracle.scan(x, delta, A, B, C, D, want_h_last=True)
    u = x.astype(np.float64)[..., None] * B.astype(np.float64)[:, :, None, :]   # (Bs, L, ED, N)
    h = np.cumsum(u, axis=1)
    y_ref = (h * C.astype(np.float64)[:, :, None, :]).sum(-1) + D * x
    assert np.array_equal(y, y_ref)
    assert np.array_equal(h_last, h[:, -1])


# --- Pin 5: special cases and invariants --------------------------------------
def test_zero_B_or_C_gives_skip_term_only():
    inp = small_inputs(2, 33, 5, 4, seed=5)
    for key in ("B", "C"):
        mod = dict(inp)
        mod[key] = np.zeros_like(inp[key])
        y, _, _ = oracle.scan(**mod)
        assert np.array_equal(y, inp["D"].astype(np.float64) * inp["x"].astype(np.float64))


def test_zero_x_gives_zero():
    inp = small_inputs(1, 20, 3, 4, seed=6)
    inp["x"] = np.zeros_like(inp["x"])
    y, h, _ = oracle.scan(**inp, want_h_last=True)
    assert not y.any() and not h.any()


def test_single_step():
    inp = small_inputs(3, 1, 7, 5, seed=7)
    y, h, _ = oracle.scan(**inp, want_h_last=True)
    d, x = inp["delta"].astype(np.float64), inp["x"].astype(np.float64)
    CB = (inp["C"].astype(np.float64) * inp["B"].astype(np.float64)).sum(-1)   # (Bs, 1)
    y_ref = d * x * CB[:, :, None] + inp["D"] * x
    assert rel_err(y, y_ref) < 1e-14
    h_ref = (d * x)[:, 0, :, None] * inp["B"].astype(np.float64)[:, 0, None, :]
    assert rel_err(h, h_ref) < 1e-15


def test_constant_inputs_geometric_series():
    # constant a and b: h_t = b (1 - a^(t+1)) / (1 - a)
    Bs, L, ED, N = 1, 300, 2, 3
    x = np.full((Bs, L, ED), 0.75, np.float32)
    delta = np.full((Bs, L, ED), 0.03125, np.float32)
    A = -np.array([[1.0, 2.0, 5.0], [0.5, 3.0, 9.0]], np.float32)
    B = np.tile(np.array([1.0, -2.0, 0.5], np.float32), (Bs, L, 1))
    C = np.tile(np.array([0.25, 1.0, -1.5], np.float32), (Bs, L, 1))
    y, h, _ = oracle.scan(x, delta, A, B, C, None, want_h_last=True)
    t = np.arange(L, dtype=np.float64)[:, None, None]
    a = np.exp(0.03125 * A.astype(np.float64))[None]            # (1, ED, N)
    b = (0.03125 * 0.75) * B[0, 0].astype(np.float64)[None, None, :]
    hs = b * (1 - a ** (t + 1)) / (1 - a)                       # (L, ED, N)
    y_ref = (hs * C[0, 0].astype(np.float64)).sum(-1)[None]
    assert rel_err(y, y_ref) < 1e-13
    assert rel_err(h[0], hs[-1]) < 1e-13


def test_stable_regime_is_bounded():
    # delta > 0 and A < 0 give 0 < a < 1: the state stays below max|b| / (1 - max a).
    # A sign slip in the exponent makes it grow without bound.
    Bs, L, ED, N = 1, 4096, 2, 16
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=11)
    _, h, _ = oracle.scan(**inp, want_h_last=True)
    d = inp["delta"].astype(np.float64)
    bmax = np.max(np.abs(d * inp["x"])[..., None] * np.abs(inp["B"]).max(), axis=1)  # (Bs, ED, 1)
    amax = np.exp(d.min(axis=1)[..., None] * inp["A"].astype(np.float64)[None])       # (Bs, ED, N)
    assert np.all(np.abs(h) <= bmax / (1 - amax) + 1e-12)


def test_linear_in_x():
    inp = small_inputs(2, 30, 4, 5, seed=12)
    x2 = synth.normal(99, 1, inp["x"].shape)
    y1, _, _ = oracle.scan(**inp)
    y2, _, _ = oracle.scan(**dict(inp, x=x2))
    y12, _, _ = oracle.scan(**dict(inp, x=(inp["x"].astype(np.float64) + x2).astype(np.float32)))
    # x1 + x2 rounds in fp32; compare against the exactly summed inputs' scan instead
    xs = (inp["x"].astype(np.float64) + x2).astype(np.float32)
    assert rel_err(y12, oracle.scan(**dict(inp, x=xs))[0]) == 0.0
    assert rel_err(y1 + y2, y12) < 1e-6


def test_missing_D_is_zero_D():
    inp = small_inputs(1, 17, 3, 4, seed=13)
    y0, _, _ = oracle.scan(**dict(inp, D=None))
    yz, _, _ = oracle.scan(**dict(inp, D=np.zeros_like(inp["D"])))
    assert np.array_equal(y0, yz)


# --- bidirectional variant -----------------------------------------------------
def test_bidir_equals_forward_plus_flipped_forward():
    # y_bidir = forward scan + flip(forward scan of flipped inputs) + D x,
    # with the flip done as an explicit copy here (the oracle reads in place).
    inp = small_inputs(2, 37, 5, 6, seed=14)
    yb, hb, gb = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True)
    yf, hf, _ = oracle.scan(**dict(inp, D=None), want_h_last=True)
    flip = {k: (np.ascontiguousarray(v[:, ::-1]) if k in ("x", "delta", "B", "C") else v)
            for k, v in inp.items()}
    yr, hr, _ = oracle.scan(**dict(flip, D=None), want_h_last=True)
    y_ref = yf + yr[:, ::-1] + inp["D"].astype(np.float64) * inp["x"].astype(np.float64)
    assert rel_err(yb, y_ref) < 1e-13
    assert np.array_equal(hb, hf)
    assert rel_err(gb, hr) < 1e-14


def test_bidir_reverse_closed_form():
    # g_t = sum_{s >= t} (prod_{r=t}^{s-1} a_r) b_s: the current step's own a_t is
    # not applied to b_t (no shift), the diagonal counts in both directions.
    Bs, L, ED, N = 1, 9, 2, 3
    inp = small_inputs(Bs, L, ED, N, seed=15)
    yb, _, _ = oracle.scan(**inp, bidir=True)
    a, b = discretise(inp["x"], inp["delta"], inp["A"], inp["B"])
    h = np.zeros_like(b)
    g = np.zeros_like(b)
    for t in range(L):
        for s in range(L):
            if s <= t:
                w = np.prod(a[s + 1:t + 1], axis=0) if t > s else np.ones_like(a[0])
                h[t] += w * b[s]
            if s >= t:
                w = np.prod(a[t:s], axis=0) if s > t else np.ones_like(a[0])
                g[t] += w * b[s]
    assert rel_err(yb, contract(h + g, inp["C"], inp["x"], inp["D"])) < 1e-13


# --- resume: final state of a split sequence ----------------------------------
def test_final_state_composes_over_a_split():
    inp = small_inputs(2, 60, 4, 5, seed=16)
    L1 = 23
    _, h_full, _ = oracle.scan(**inp, want_h_last=True)
    pre = {k: (np.ascontiguousarray(v[:, :L1]) if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    suf = {k: (np.ascontiguousarray(v[:, L1:]) if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    _, h1, _ = oracle.scan(**pre, want_h_last=True)
    _, h2, _ = oracle.scan(**suf, want_h_last=True)
    a, _ = discretise(suf["x"], suf["delta"], suf["A"], suf["B"])
    P = np.prod(a, axis=0)                                   # (Bs, ED, N)
    assert rel_err(h_full, P * h1 + h2) < 1e-13


# --- dtype and plumbing -------------------------------------------------------
def test_bf16_inputs_widen_exactly():
    inp = synth.make_inputs(2, 40, 8, 16, "bf16", seed=17)
    y, h, _ = oracle.scan(**inp, want_h_last=True)
    wide = {k: (synth.from_bf16(v) if v.dtype == np.uint16 else v) for k, v in inp.items()}
    y2, h2, _ = oracle.scan(**wide, want_h_last=True)
    assert np.array_equal(y, y2) and np.array_equal(h, h2)


def test_channel_subset_and_threads_agree():
    inp = small_inputs(3, 45, 7, 4, seed=18)
    y, h, _ = oracle.scan(**inp, want_h_last=True, nthreads=1)
    y8, h8, _ = oracle.scan(**inp, want_h_last=True, nthreads=8)
    assert np.array_equal(y, y8) and np.array_equal(h, h8)
    chans = np.array([0, 20, 7, 13], np.int64)
    ys, hs, _ = oracle.scan(**inp, chans=chans, want_h_last=True)
    for k, c in enumerate(chans):
        b, e = divmod(int(c), 7)
        assert np.array_equal(ys[k], y[b, :, e])
        assert np.array_equal(hs[k], h[b, e])


def test_oracle_rejects_bad_arguments():
    inp = small_inputs(1, 4, 2, 2)
    with pytest.raises(RuntimeError):
        oracle.scan(**inp, chans=np.array([5], np.int64))


# --- initial state: resuming a split sequence ----------------------------------
def test_initial_state_superposition_and_resume():
    # the scan is affine in its initial state: starting [L1, L) from h0 adds
    # sum_n C_t[n] (prod_{s<=t} a_s[n]) h0[n] to y and (prod a) h0 to h_L;
    # with h0 = the carried state h_{L1-1} it resumes the full scan
    inp = small_inputs(2, 70, 5, 16, seed=23)
    L1 = 29
    pre = {k: (np.ascontiguousarray(v[:, :L1]) if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    suf = {k: (np.ascontiguousarray(v[:, L1:]) if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    y_full, h_full, _ = oracle.scan(**inp, want_h_last=True)
    _, h1, _ = oracle.scan(**pre, want_h_last=True)
    h0 = h1.astype(np.float32)   # the initial-state input is float32
    y2, h2, _ = oracle.scan(**suf, h0=h0, want_h_last=True)
    y_ref, h_ref, _ = oracle.scan(**suf, want_h_last=True)
    a, _ = discretise(suf["x"], suf["delta"], suf["A"], suf["B"])
    P = np.cumprod(a, axis=0)                                   # (L2, Bs, ED, N)
    Ct = suf["C"].astype(np.float64).transpose(1, 0, 2)[:, :, None, :]
    corr = (P * h0.astype(np.float64)[None] * Ct).sum(-1).transpose(1, 0, 2)
    assert rel_err(y2, y_ref + corr) < 1e-13
    assert rel_err(h2, h_ref + P[-1] * h0) < 1e-13
    # resuming from the (float32-rounded) carried state reproduces the full scan
    assert rel_err(y2, y_full[:, L1:]) < 1e-6


def test_zero_initial_state_is_no_initial_state():
    inp = small_inputs(2, 31, 4, 16, seed=24)
    y0, h0_, _ = oracle.scan(**inp, want_h_last=True)
    yz, hz, _ = oracle.scan(**inp, h0=np.zeros((2, 4, 16), np.float32), want_h_last=True)
    assert np.array_equal(y0, yz) and np.array_equal(h0_, hz)


def test_empty_sequence_keeps_the_entering_state():
    # zero steps: no output, the forward state stays h0 (or zero) and the
    # reverse state g_L = 0; a sequence cut at L1 = 0 resumes exactly
    inp = small_inputs(2, 37, 5, 16, seed=25)
    empty = {k: (np.ascontiguousarray(v[:, :0]) if k in ("x", "delta", "B", "C") else v) for k, v in inp.items()}
    h0 = (0.5 * synth.normal(25, 9, (2, 5, 16))).astype(np.float32)
    y, h, g = oracle.scan(**empty, h0=h0, bidir=True, want_h_last=True, want_g_first=True)
    assert y.shape == (2, 0, 5)
    assert np.array_equal(h, h0.astype(np.float64)) and np.array_equal(g, np.zeros((2, 5, 16)))
    _, hz, _ = oracle.scan(**empty, want_h_last=True)
    assert np.array_equal(hz, np.zeros((2, 5, 16)))
    y_full, h_full, _ = oracle.scan(**inp, h0=h0, want_h_last=True)
    y2, h2, _ = oracle.scan(**inp, h0=h.astype(np.float32), want_h_last=True)
    assert np.array_equal(y2, y_full) and np.array_equal(h2, h_full)


def test_empty_batch_or_channels_give_empty_outputs():
    for Bs, ED in ((0, 5), (2, 0)):
        inp = small_inputs(Bs, 9, ED, 16, seed=26) if Bs * ED else synth.make_inputs(Bs, 9, ED, 16, seed=26)
        y, h, g = oracle.scan(**inp, bidir=True, want_h_last=True, want_g_first=True)
        assert y.shape == (Bs, 9, ED) and h.shape == (Bs, ED, 16) and g.shape == (Bs, ED, 16)


# --- step-size pre-processing and the output gate -----------------------------
def test_dt_bias_is_added_to_delta_exactly():
    # delta and bias on a 2^-12 grid: delta + bias is exact in float32, so the
    # biased scan must equal the scan of the pre-added step sizes bitwise
    inp = small_inputs(2, 40, 6, 16, seed=25)
    rng = np.random.default_rng(25)
    inp["delta"] = (rng.integers(1, 200, inp["delta"].shape) / 4096.0).astype(np.float32)
    bias = (rng.integers(-20, 40, (6,)) / 4096.0).astype(np.float32)
    y1, h1, _ = oracle.scan(**inp, dt_bias=bias, want_h_last=True)
    y2, h2, _ = oracle.scan(**dict(inp, delta=(inp["delta"] + bias).astype(np.float32)), want_h_last=True)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_softplus_step_sizes():
    # softplus(v) = log(1 + e^v): against step sizes transformed with numpy
    # (rounded to float32, hence the tolerance), and softplus(0) = ln 2
    inp = small_inputs(2, 50, 5, 16, seed=26)
    raw = synth.normal(26, 11, inp["delta"].shape) * 2.0 - 3.0
    y1, _, _ = oracle.scan(**dict(inp, delta=raw.astype(np.float32)), dt_softplus=True)
    sp = np.log1p(np.exp(raw.astype(np.float32).astype(np.float64))).astype(np.float32)
    y2, _, _ = oracle.scan(**dict(inp, delta=sp))
    assert rel_err(y1, y2) < 1e-6
    zero = np.zeros_like(inp["delta"])
    y3, _, _ = oracle.scan(**dict(inp, delta=zero), dt_softplus=True)
    y4, _, _ = oracle.scan(**dict(inp, delta=np.full_like(zero, np.log(2.0))))
    assert rel_err(y3, y4) < 1e-7
    big = np.full_like(zero, 30.0)   # above the threshold softplus is the identity
    y5, _, _ = oracle.scan(**dict(inp, delta=big), dt_softplus=True)
    y6, _, _ = oracle.scan(**dict(inp, delta=big))
    assert np.array_equal(y5, y6)


def test_dt_limit_clamps():
    inp = small_inputs(1, 60, 4, 16, seed=27)
    lo, hi = 0.0078125, 0.046875   # float32-representable bounds
    y1, _, _ = oracle.scan(**inp, dt_limit=(lo, hi))
    y2, _, _ = oracle.scan(**dict(inp, delta=np.clip(inp["delta"], np.float32(lo), np.float32(hi))))
    assert rel_err(y1, y2) < 1e-15


def test_gate_special_values():
    inp = small_inputs(2, 30, 4, 16, seed=28)
    y, _, _ = oracle.scan(**inp)
    zero = np.zeros_like(inp["x"])
    yz, _, _ = oracle.scan(**inp, z=zero)                    # silu(0) = 0
    assert not yz.any()
    yb, _, _ = oracle.scan(**inp, z=np.full_like(zero, 50.0))  # sigmoid(50) = 1 in double
    assert rel_err(yb, 50.0 * y) < 1e-15
    yn, _, _ = oracle.scan(**inp, z=np.full_like(zero, -800.0))  # e^800 overflows: exact zero
    assert not yn.any()
    yo, _, _ = oracle.scan(**inp, z=np.ones_like(zero))       # silu(1) = 1 / (1 + 1/e)
    assert rel_err(yo, y / (1.0 + np.exp(-1.0))) < 1e-15


def test_gate_and_bias_apply_to_bidirectional_output():
    inp = small_inputs(2, 33, 4, 16, seed=29)
    z = synth.normal(29, 12, inp["x"].shape)
    bias = synth.normal(29, 13, (4,)) * 0.01
    yb, _, _ = oracle.scan(**inp, bidir=True, dt_bias=bias, dt_softplus=True, z=z)
    sp = np.log1p(np.exp(inp["delta"].astype(np.float64) + bias.astype(np.float64)))
    yu, _, _ = oracle.scan(**dict(inp, delta=sp.astype(np.float32)), bidir=True)
    g = z.astype(np.float64) / (1.0 + np.exp(-z.astype(np.float64)))
    assert rel_err(yb, yu * g) < 1e-6

"""fp64 CPU oracle for the selective scan (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its binding) never does.

``scan`` is the sequential definition written out in ``ssm_oracle.c``:
  a_t[n] = exp(delta_t * A[e, n]);  h_t = a_t * h_{t-1} + (delta_t * x_t) * B_t[n]
  y_t = sum_n C_t[n] h_t[n] + D[e] x_t
(plus the reverse-time scan for the bidirectional variant), in fp64.
``scan_bwd`` is the adjoint of that recurrence: the gradients of sum(dy * y)
with respect to x, delta, A, B, C, D and h0. ``ssd`` is the multi-head
(Mamba-2 / SSD) form: one scalar decay per head, B and C shared by a group of
heads, a (headdim x state) matrix state per head.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_SO = os.path.join(_HERE, "libssm_oracle.so")
_lib = None

F32, BF16 = 0, 1


def build():
    """Compile the oracle with gcc (no fast-math: IEEE fp64 throughout)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        dbl = ctypes.c_double
        L.oracle_scan.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, ctypes.c_int, dbl, dbl, vp,
                                  i64, i64, i64, i64, vp, i64, vp, vp, vp, ctypes.c_int]
        L.oracle_scan.restype = ctypes.c_int
        L.oracle_scan_bwd.argtypes = ([ctypes.c_int] + [vp] * 9 + [ctypes.c_int, ctypes.c_double, ctypes.c_double] +
                                      [vp] * 2 + [i64] * 4 + [vp] * 8 + [ctypes.c_int])
        L.oracle_scan_bwd.restype = ctypes.c_int
        L.oracle_ssd.argtypes = ([ctypes.c_int, ctypes.c_int] + [vp] * 9 + [ctypes.c_int, ctypes.c_double,
                                 ctypes.c_double, vp] + [i64] * 6 + [vp] * 3 + [ctypes.c_int])
        L.oracle_ssd.restype = ctypes.c_int
        _lib = L
    return _lib


def _threads(nthreads):
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    return int(nthreads)


def _ptr(a):
    return None if a is None else a.ctypes.data


def scan(x, delta, A, B, C, D=None, *, h0=None, g0=None, dt_bias=None, dt_softplus=False,
         dt_limit=(-float("inf"), float("inf")), z=None, bidir=False, chans=None, want_h_last=False,
         want_g_first=False, nthreads=None):
    """Run the oracle.

    x, delta: (Bs, L, ED); B, C: (Bs, L, N) -- float32, or uint16 bf16 bit
    patterns (all four the same dtype). A: (ED, N) float32; D: (ED,) float32
    or None. h0: optional (Bs, ED, N) float32 initial forward state (zero if
    None). dt_bias (ED,) float32, dt_softplus, dt_limit = (lo, hi): the step
    size used is clamp(softplus?(delta + dt_bias), lo, hi) (no clamp by
    default: raw step sizes may be negative). z: optional gate,
    same shape and dtype as x; the output is multiplied by z * sigmoid(z).
    chans: optional int64 array of channel ids b*ED + e.

    Returns (y, h_last, g_first): y is (Bs, L, ED) float64 when chans is None,
    else (len(chans), L) channel-major; h_last / g_first are (Bs, ED, N) or
    (len(chans), N), or None when not requested.
    """
    x = np.ascontiguousarray(x)
    delta = np.ascontiguousarray(delta)
    B = np.ascontiguousarray(B)
    C = np.ascontiguousarray(C)
    A = np.ascontiguousarray(A, dtype=np.float32)
    D = None if D is None else np.ascontiguousarray(D, dtype=np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float32)
    g0 = None if g0 is None else np.ascontiguousarray(g0, dtype=np.float32)
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
    z = None if z is None else np.ascontiguousarray(z)
    if z is not None and (z.dtype != x.dtype or z.shape != x.shape):
        raise TypeError("z must match x in shape and dtype")
    if x.dtype == np.uint16:
        dtype = BF16
    elif x.dtype == np.float32:
        dtype = F32
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    for t in (delta, B, C):
        if t.dtype != x.dtype:
            raise TypeError("x, delta, B, C must share a dtype")
    Bs, L, ED = x.shape
    N = A.shape[1]
    assert delta.shape == x.shape and B.shape == (Bs, L, N) and C.shape == (Bs, L, N)
    assert A.shape == (ED, N) and (D is None or D.shape == (ED,))
    assert h0 is None or h0.shape == (Bs, ED, N)
    assert g0 is None or g0.shape == (Bs, ED, N)
    assert dt_bias is None or dt_bias.shape == (ED,)
    if chans is not None:
        chans = np.ascontiguousarray(chans, dtype=np.int64)
        nch = chans.size
    else:
        nch = Bs * ED
    y = np.empty((nch, L), dtype=np.float64)
    h = np.empty((nch, N), dtype=np.float64) if want_h_last else None
    g = np.empty((nch, N), dtype=np.float64) if (want_g_first and bidir) else None
    rc = lib().oracle_scan(dtype, int(bool(bidir)), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                           _ptr(D), _ptr(h0), _ptr(g0), _ptr(dt_bias), int(bool(dt_softplus)), float(dt_limit[0]),
                           float(dt_limit[1]), _ptr(z), Bs, L, ED, N, _ptr(chans), nch, _ptr(y), _ptr(h), _ptr(g),
                           _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_scan failed with code %d" % rc)
    if chans is None:
        y = y.reshape(Bs, ED, L).transpose(0, 2, 1)
        if h is not None:
            h = h.reshape(Bs, ED, N)
        if g is not None:
            g = g.reshape(Bs, ED, N)
    return y, h, g


def scan_bwd(x, delta, A, B, C, D=None, dy=None, *, h0=None, g0=None, dh_last=None, dg_first=None, dt_bias=None,
             dt_softplus=False, dt_limit=(-float("inf"), float("inf")), z=None, bidir=False, nthreads=None):
    """Gradients of L = sum(dy * y) for the forward scan, in fp64.

    Same input conventions as scan() (including the options dt_bias,
    dt_softplus, dt_limit and the gate z); dy has y's shape and x's dtype.
    Returns a dict with dx, ddelta (Bs, L, ED; ddelta is the gradient of the
    raw step size, through the step-size map), dA (ED, N), dB, dC (Bs, L, N),
    dD (ED,) and dh0 (Bs, ED, N) (the same with or without h0: y is affine in
    the initial state), and ddt_bias (ED,) when dt_bias is given, dz (like x)
    when z is given.

    With a gate, y' = y z sigmoid(z): the scan itself sees the output
    gradient dy z sigmoid(z), and dz = dy y (d/dz of z sigmoid(z)) with y the
    whole ungated output (both directions and D x), taken from scan().

    dh_last: optional (Bs, ED, N) gradient of the loss with respect to the
    final state h_last (the Bi-Mamba2 backward's dfinal_states): the loss is
    then sum(dy * y) + sum(dh_last * h_last).

    bidir: the gradients of the bidirectional scan, whose output is the
    forward scan (with D x and h0) plus the reverse-time scan, i.e. the
    forward scan of the time-flipped inputs from g0 (zero if None) without D,
    flipped back ("Some questions of Bi-Mamba2 and Hydra", the author's first
    reply). Its gradient is the sum of the two scans' gradients, the reverse
    one taken on flipped copies and flipped back; D and h0 enter the forward
    scan only, g0 the reverse one; the step-size map and the gate's factor
    apply to both. dg_first (the gradient of the reverse final state g_first)
    enters the reverse scan's adjoint as dh_last enters the forward one, and
    the result holds dg0 (the gradient of g0) beside dh0.
    """
    opts = dict(dt_bias=dt_bias, dt_softplus=dt_softplus, dt_limit=dt_limit)
    if bidir:
        fwd = scan_bwd(x, delta, A, B, C, D, dy, h0=h0, dh_last=dh_last, z=z, nthreads=nthreads, **opts)
        flip = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])
        rev = scan_bwd(flip(x), flip(delta), A, flip(B), flip(C), None, flip(dy), h0=g0, dh_last=dg_first,
                       z=None if z is None else flip(z), nthreads=nthreads, **opts)
        for k in ("dx", "ddelta", "dB", "dC"):
            fwd[k] = fwd[k] + rev[k][:, ::-1]
        fwd["dA"] = fwd["dA"] + rev["dA"]
        fwd["dg0"] = rev["dh0"]
        if dt_bias is not None:
            fwd["ddt_bias"] = fwd["ddt_bias"] + rev["ddt_bias"]
        if z is not None:
            fwd["dz"] = _gate_grad(x, delta, A, B, C, D, dy, h0, z, True, nthreads, opts, g0=g0)
        return fwd
    if g0 is not None or dg_first is not None:
        raise ValueError("g0 and dg_first belong to the bidirectional scan")
    x = np.ascontiguousarray(x)
    delta = np.ascontiguousarray(delta)
    B = np.ascontiguousarray(B)
    C = np.ascontiguousarray(C)
    dy = np.ascontiguousarray(dy)
    A = np.ascontiguousarray(A, dtype=np.float32)
    D = None if D is None else np.ascontiguousarray(D, dtype=np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float32)
    dhl = None if dh_last is None else np.ascontiguousarray(dh_last, dtype=np.float32)
    dtb = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
    zc = None if z is None else np.ascontiguousarray(z)
    dtype = BF16 if x.dtype == np.uint16 else F32
    for t in (delta, B, C, dy) + (() if zc is None else (zc,)):
        if t.dtype != x.dtype:
            raise TypeError("x, delta, B, C, dy (and z) must share a dtype")
    Bs, L, ED = x.shape
    N = A.shape[1]
    assert dy.shape == x.shape and (zc is None or zc.shape == x.shape)
    assert dtb is None or dtb.shape == (ED,)
    assert dhl is None or dhl.shape == (Bs, ED, N)
    out = dict(dx=np.empty((Bs, L, ED)), ddelta=np.empty((Bs, L, ED)), dA=np.empty((ED, N)),
               dB=np.empty((Bs, L, N)), dC=np.empty((Bs, L, N)), dD=np.empty((ED,)), dh0=np.empty((Bs, ED, N)))
    dbias = np.empty((ED,)) if dtb is not None else None
    rc = lib().oracle_scan_bwd(dtype, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dhl),
                               _ptr(dtb),
                               int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]), _ptr(zc), _ptr(dy),
                               Bs, L, ED, N, _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
                               _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]), _ptr(dbias), _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_scan_bwd failed with code %d" % rc)
    if dbias is not None:
        out["ddt_bias"] = dbias
    if zc is not None:
        out["dz"] = _gate_grad(x, delta, A, B, C, D, dy, h0, zc, False, nthreads, opts)
    return out


def _gate_grad(x, delta, A, B, C, D, dy, h0, z, bidir, nthreads, opts, g0=None):
    """dz = dy y d(z sigmoid(z))/dz for y' = y z sigmoid(z), with y the
    ungated output of the scan (forward or bidirectional, with the options)."""
    y, _, _ = scan(x, delta, A, B, C, D, h0=h0, g0=g0, bidir=bidir, nthreads=nthreads, **opts)
    zf = _widen(z)
    sg = 1.0 / (1.0 + np.exp(-zf))
    return _widen(dy) * y * (sg * (1.0 + zf * (1.0 - sg)))


def _widen(a):
    """float32 or bf16 (uint16 bits) -> float64"""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ssd(x, dt, A, B, C, D=None, *, h0=None, g0=None, dt_bias=None, dt_softplus=False,
        dt_limit=(-float("inf"), float("inf")), z=None, bidir=False, want_h_last=False, want_g_first=False,
        nthreads=None):
    """Multi-head selective scan in fp64.

    x (Bs, L, H, P), dt (Bs, L, H), A (H,), B and C (Bs, L, G, N), D (H,) or
    None, h0 (Bs, H, P, N) or None, g0 (Bs, H, P, N) or None (the reverse
    state entering at the last step, bidir only); float32 arrays, or uint16 bfloat16 bit
    patterns for x, dt, B, C. dt_bias (H,) float32, dt_softplus, dt_limit and
    the gate z (x's shape and dtype) as in scan(), per head. Returns
    (y (Bs, L, H, P), h_last, g_first) with the states (Bs, H, P, N) when
    requested, else None.
    """
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
    z = None if z is None else np.ascontiguousarray(z)
    if z is not None and (z.dtype != np.asarray(x).dtype or z.shape != np.shape(x)):
        raise TypeError("z must match x in shape and dtype")
    x = np.ascontiguousarray(x)
    dt = np.ascontiguousarray(dt)
    B = np.ascontiguousarray(B)
    C = np.ascontiguousarray(C)
    A = np.ascontiguousarray(A, dtype=np.float32)
    D = None if D is None else np.ascontiguousarray(D, dtype=np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float32)
    g0 = None if g0 is None else np.ascontiguousarray(g0, dtype=np.float32)
    dtype = BF16 if x.dtype == np.uint16 else F32
    for t in (dt, B, C):
        if t.dtype != x.dtype:
            raise TypeError("x, dt, B, C must share a dtype")
    Bs, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bs, L, H) and B.shape == C.shape == (Bs, L, G, N) and A.shape == (H,)
    assert dt_bias is None or dt_bias.shape == (H,)
    y = np.empty((Bs, L, H, P))
    hl = np.empty((Bs, H, P, N)) if want_h_last else None
    gf = np.empty((Bs, H, P, N)) if (want_g_first and bidir) else None
    assert g0 is None or g0.shape == (Bs, H, P, N)
    rc = lib().oracle_ssd(dtype, int(bool(bidir)), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                          _ptr(g0),
                          _ptr(dt_bias), int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]), _ptr(z),
                          Bs, L, H, P, G, N, _ptr(y), _ptr(hl), _ptr(gf), _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_ssd failed with code %d" % rc)
    return y, hl, gf

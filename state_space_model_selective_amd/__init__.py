"""Python binding of the MI355X selective-scan library (libssm_scan.so).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``csrc/ssm_scan.hip`` (forward), ``csrc/ssm_scan_bwd.hip`` (backward) and
``csrc/ssm_ssd.hip`` (multi-head scan) behind the C ABI declared in
``include/ssm_scan.h``.
PyTorch supplies device memory and the stream. There is no fallback: if the
library is not built, or the tensors are not on a GPU, the calls raise.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libssm_scan.so")
SOURCES = [os.path.join(_HERE, "csrc", n) for n in ("ssm_scan.hip", "ssm_scan_bwd.hip", "ssm_ssd.hip")]
# issue-rate probe of the vector ALU (measurement only; used by the benchmark's --micro mode)
PROBE_LIB_PATH = os.path.join(_HERE, "libssm_valu_probe.so")
PROBE_SOURCES = [os.path.join(_HERE, "csrc", "valu_probe.hip")]
INCLUDE = os.path.join(_ROOT, "include")

SSM_F32, SSM_BF16 = 0, 1
# bytes of the device buffer that ssm_scan_fwd_noalloc uses in place of a workspace
SSM_NOALLOC_SCRATCH_BYTES = 1 << 20
(SSM_OK, SSM_ERR_NULL, SSM_ERR_DIM, SSM_ERR_UNSUPPORTED, SSM_ERR_ALIAS, SSM_ERR_WORKSPACE, SSM_ERR_LAUNCH,
 SSM_ERR_ARG, SSM_ERR_HANDOFF) = range(9)


class SSMOptions(ctypes.Structure):
    """ssm_scan_options: step-size pre-processing and output gate."""
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float), ("z", ctypes.c_void_p)]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # no packed-FP32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

_lib = None
_probe = None


class SSMError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_str(status), status))


def _hipcc(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", INCLUDE] + sources + ["-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout)
    if verbose:
        print(res.stdout)
    os.replace(tmp, out)


def build(verbose=False):
    """Compile libssm_scan.so (and the ALU issue-rate probe) for gfx950 with
    hipcc (works without a GPU)."""
    _hipcc(SOURCES, LIB_PATH, verbose)
    _hipcc(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    global _lib, _probe
    _lib = None
    _probe = None


def _load_torch_runtime():
    """Import torch before the library is loaded: the library's HIP runtime
    dependency then binds to the runtime torch has loaded, so that one runtime
    serves torch's memory and streams and the library's launches (loaded
    first, the system runtime would take that name and torch's own would
    fail to find a device)."""
    import torch  # noqa: F401


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssm_scan.so is not built (run __graft_entry__.build())")
        _load_torch_runtime()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        L.ssm_scan_workspace_bytes.argtypes = [i64, i64, i64, i64, ci, ci]
        L.ssm_scan_workspace_bytes.restype = sz
        L.ssm_scan_fwd.argtypes = [vp] * 10 + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_fwd.restype = ci
        L.ssm_scan_bidir_fwd.argtypes = [vp] * 12 + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_bidir_fwd.restype = ci
        L.ssm_scan_ckpt_bytes.argtypes = [i64] * 4
        L.ssm_scan_ckpt_bytes.restype = sz
        L.ssm_scan_fwd_ckpt.argtypes = [vp] * 11 + [sz] + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_fwd_ckpt.restype = ci
        L.ssm_scan_bwd_ckpt.argtypes = [vp] * 11 + [sz] + [vp] * 9 + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_bwd_ckpt.restype = ci
        L.ssm_scan_fwd_status.argtypes = [vp, sz] + [i64] * 4 + [ci, vp]
        L.ssm_scan_fwd_status.restype = ci
        L.ssm_scan_fwd_noalloc.argtypes = [vp] * 10 + [i64] * 4 + [ci, vp]
        L.ssm_scan_fwd_noalloc.restype = ci
        L.ssm_scan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci, ci]
        L.ssm_scan_bwd_workspace_bytes.restype = sz
        L.ssm_scan_bwd.argtypes = [vp] * 19 + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_bwd.restype = ci
        L.ssm_scan_bidir_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci, ci]
        L.ssm_scan_bidir_bwd_workspace_bytes.restype = sz
        L.ssm_scan_bidir_bwd.argtypes = [vp] * 22 + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_bidir_bwd.restype = ci
        L.ssm_scan_bidir_fwd_ckpt.argtypes = [vp] * 13 + [sz] + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_bidir_fwd_ckpt.restype = ci
        L.ssm_scan_bidir_bwd_ckpt.argtypes = [vp] * 13 + [sz] + [vp] * 10 + [i64] * 4 + [ci, vp, sz, vp]
        L.ssm_scan_bidir_bwd_ckpt.restype = ci
        L.ssm_ssd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
        L.ssm_ssd_workspace_bytes.restype = sz
        L.ssm_ssd_fwd.argtypes = [vp] * 10 + [i64] * 6 + [ci, vp, sz, vp]
        L.ssm_ssd_fwd.restype = ci
        L.ssm_ssd_bidir_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
        L.ssm_ssd_bidir_workspace_bytes.restype = sz
        L.ssm_ssd_bidir_fwd.argtypes = [vp] * 12 + [i64] * 6 + [ci, vp, sz, vp]
        L.ssm_ssd_bidir_fwd.restype = ci
        L.ssm_status_str.argtypes = [ci]
        L.ssm_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def probe_lib():
    """The ALU issue-rate probe library (measurement only)."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError("libssm_valu_probe.so is not built (run __graft_entry__.build())")
        _load_torch_runtime()
        P = ctypes.CDLL(PROBE_LIB_PATH)
        P.ssm_probe_valu_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]
        P.ssm_probe_valu_launch.restype = ctypes.c_int
        P.ssm_probe_valu_ops_per_iter.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                                  ctypes.POINTER(ctypes.c_int)]
        P.ssm_probe_valu_ops_per_iter.restype = ctypes.c_int
        _probe = P
    return _probe


def status_str(status):
    return lib().ssm_status_str(int(status)).decode()


def ssm_scan_workspace_bytes(Bs, L, ED, N, dtype=SSM_F32, bidir=False):
    return int(lib().ssm_scan_workspace_bytes(Bs, L, ED, N, int(dtype), int(bool(bidir))))


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("x must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


class _Args:
    """Checks every tensor of one call against x (dtype, shape, contiguity,
    device) before any pointer is taken: the C ABI sees only addresses and
    sizes, so a tensor of the wrong dtype, shape or layout would be misread
    there. The GPU check comes last (check_gpu), so that each rejection also
    shows on CPU tensors."""

    def __init__(self, where, x, ndim):
        import torch
        self.where = where
        if not isinstance(x, torch.Tensor):
            raise TypeError("%s: x must be a torch.Tensor, got %s" % (where, type(x).__name__))
        if x.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("%s: x must be float32 or bfloat16, got %s" % (where, x.dtype))
        if x.dim() != ndim:
            raise ValueError("%s: x must have %d dimensions, got shape %s" % (where, ndim, tuple(x.shape)))
        self.x = x
        self.dtype = x.dtype
        self.device = x.device
        self.check("x", x, tuple(x.shape))

    def check(self, name, t, shape, dtype=None, required=False):
        """t may be None unless required; dtype None means x's dtype."""
        import torch
        if t is None:
            if required:
                raise ValueError("%s: %s is required" % (self.where, name))
            return
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: %s must be a torch.Tensor, got %s" % (self.where, name, type(t).__name__))
        want = self.dtype if dtype is None else dtype
        if t.dtype != want:
            raise TypeError("%s: %s must be %s, got %s" % (self.where, name, want, t.dtype))
        if t.device != self.device:
            raise ValueError("%s: %s is on %s, x on %s" % (self.where, name, t.device, self.device))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s: %s must have shape %s, got %s" % (self.where, name, tuple(shape), tuple(t.shape)))
        if not t.is_contiguous():
            raise ValueError("%s: %s must be contiguous (dense row-major)" % (self.where, name))

    def matrix(self, name, t, rows):
        """A 2-D float32 tensor with `rows` rows; returns its column count."""
        import torch
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError("%s: %s must be a 2-D tensor" % (self.where, name))
        self.check(name, t, (rows, t.shape[1]), torch.float32, required=True)
        return int(t.shape[1])

    def workspace(self, t):
        import torch
        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: workspace must be a torch.Tensor" % self.where)
        if t.device != self.device:
            raise ValueError("%s: workspace is on %s, x on %s" % (self.where, t.device, self.device))
        if not t.is_contiguous():
            raise ValueError("%s: workspace must be contiguous" % self.where)

    def limit(self, dt_limit):
        if dt_limit is None:
            return
        if len(dt_limit) != 2:
            raise ValueError("%s: dt_limit must be a pair (lo, hi)" % self.where)

    def check_gpu(self):
        if not self.x.is_cuda:
            raise RuntimeError("the selective scan runs on the GPU only; x is on %s" % self.x.device)


def _scan_args(where, x, delta, A, B, C, D, h0, dt_bias, dt_limit, z, workspace, outs):
    """Validates the per-channel scan's arguments; returns (checker, dims).
    outs: (name, tensor, kind[, required]) with kind 'seq' (like x), 'bc'
    (like B), 'state' (Bs, ED, N) float32, 'ed' (ED,) float32, 'a' (ED, N)
    float32, 'ckpt' the round checkpoints (float32)."""
    import torch
    a = _Args(where, x, 3)
    Bs, L, ED = (int(v) for v in x.shape)
    N = a.matrix("A", A, ED)
    f32 = torch.float32
    a.check("delta", delta, (Bs, L, ED), required=True)
    a.check("B", B, (Bs, L, N), required=True)
    a.check("C", C, (Bs, L, N), required=True)
    a.check("D", D, (ED,), f32)
    a.check("h0", h0, (Bs, ED, N), f32)
    a.check("dt_bias", dt_bias, (ED,), f32)
    a.check("z", z, (Bs, L, ED))
    a.limit(dt_limit)
    shapes = {"seq": ((Bs, L, ED), None), "bc": ((Bs, L, N), None), "state": ((Bs, ED, N), f32),
              "ed": ((ED,), f32), "a": ((ED, N), f32), "ckpt": (ssm_scan_ckpt_shape(Bs, L, ED), f32)}
    for name, t, kind, *req in outs:
        shp, dt = shapes[kind]
        a.check(name, t, shp, dt, required=bool(req and req[0]))
    a.workspace(workspace)
    a.check_gpu()
    return a, (Bs, L, ED, N)


def _workspace(workspace, need, device):
    import torch
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, ws_bytes


def _options(dt_bias, dt_softplus, dt_limit, z):
    """An SSMOptions for ctypes.byref, or None when no option is set."""
    if dt_bias is None and not dt_softplus and dt_limit is None and z is None:
        return None
    lo, hi = (-float("inf"), float("inf")) if dt_limit is None else dt_limit
    return SSMOptions(_ptr(dt_bias), int(bool(dt_softplus)), float(lo), float(hi), _ptr(z))


def _byref(o):
    return None if o is None else ctypes.byref(o)


def _stream(x, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def ssm_scan_ckpt_shape(Bs, L, ED):
    """Shape of the round checkpoints (float32): (Bs, ceil(L / 32), 16 ceil(ED / 16), 16)."""
    return (Bs, (L + 31) // 32, (ED + 15) // 16 * 16, 16)


def ssm_scan_fwd(x, delta, A, B, C, D=None, y=None, h_last=None, workspace=None, stream=None, h0=None,
                 dt_bias=None, dt_softplus=False, dt_limit=None, z=None, ckpt=None):
    """y = selective_scan(x, delta, A, B, C, D) from initial state h0 (zero if None);
    optionally the final state into h_last. dt_bias / dt_softplus / dt_limit
    pre-process delta, z gates the output (y * silu(z)). With ckpt (a float32
    tensor of ssm_scan_ckpt_shape(Bs, L, ED)) the state entering every
    32-step round is written there as well (ssm_scan_fwd_ckpt), for
    ssm_scan_bwd(..., ckpt=ckpt)."""
    import torch
    _, (Bs, L, ED, N) = _scan_args("ssm_scan_fwd", x, delta, A, B, C, D, h0, dt_bias, dt_limit, z, workspace,
                                   [("y", y, "seq"), ("h_last", h_last, "state"), ("ckpt", ckpt, "ckpt")])
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    workspace, ws_bytes = _workspace(workspace, ssm_scan_workspace_bytes(Bs, L, ED, N, dt, False), x.device)
    opts = _options(dt_bias, dt_softplus, dt_limit, z)
    head = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _byref(opts), _ptr(y), _ptr(h_last))
    tail = (Bs, L, ED, N, dt, _ptr(workspace), ws_bytes, _stream(x, stream))
    if ckpt is None:
        rc = lib().ssm_scan_fwd(*head, *tail)
    else:
        rc = lib().ssm_scan_fwd_ckpt(*head, _ptr(ckpt), ckpt.numel() * 4, *tail)
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_scan_fwd_ckpt" if ckpt is not None else "ssm_scan_fwd")
    return y


def ssm_scan_fwd_noalloc(x, delta, A, B, C, D=None, y=None, h_last=None, stream=None, h0=None, dt_bias=None,
                         dt_softplus=False, dt_limit=None, z=None):
    """ssm_scan_fwd without a workspace: the library's own device buffer holds
    the split-sequence hand-off (calls that overlap in time on one device
    race). y must be given by callers that cannot allocate."""
    _scan_args("ssm_scan_fwd_noalloc", x, delta, A, B, C, D, h0, dt_bias, dt_limit, z, None,
               [("y", y, "seq"), ("h_last", h_last, "state")])
    Bs, L, ED = (int(v) for v in x.shape)
    N = int(A.shape[1])
    dt = _dtype_code(x)
    if y is None:
        import torch
        y = torch.empty_like(x)
    opts = _options(dt_bias, dt_softplus, dt_limit, z)
    rc = lib().ssm_scan_fwd_noalloc(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                                    _byref(opts), _ptr(y), _ptr(h_last), Bs, L, ED, N, dt, _stream(x, stream))
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_scan_fwd_noalloc")
    return y


def ssm_scan_fwd_status(x, A, workspace, stream=None):
    """Outcome of the split-sequence hand-off of the last ssm_scan_fwd call on
    tensors shaped like x and A with this workspace (None: the last
    ssm_scan_fwd_noalloc call on this device): synchronises the stream,
    returns SSM_OK or SSM_ERR_HANDOFF (a hand-off wait gave up; that call's
    affected outputs are NaN); raises SSMError for argument errors."""
    a = _Args("ssm_scan_fwd_status", x, 3)
    Bs, L, ED = (int(v) for v in x.shape)
    N = a.matrix("A", A, ED)
    a.workspace(workspace)
    a.check_gpu()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().ssm_scan_fwd_status(_ptr(workspace), ws_bytes, Bs, L, ED, N, _dtype_code(x), _stream(x, stream))
    if rc not in (SSM_OK, SSM_ERR_HANDOFF):
        raise SSMError(rc, "ssm_scan_fwd_status")
    return rc


def ssm_scan_bidir_fwd(x, delta, A, B, C, D=None, y=None, h_last=None, g_first=None, workspace=None,
                       stream=None, h0=None, g0=None, dt_bias=None, dt_softplus=False, dt_limit=None, z=None,
                       ckpt=None):
    """y = forward scan (from h0, zero if None) + reverse-time scan (from g0
    at the last step, zero if None; shared weights, read in place) + D x,
    with the same options as ssm_scan_fwd. With ckpt (float32, of
    ssm_scan_ckpt_shape(Bs, L, ED)) the forward direction's round states are
    written there as well (ssm_scan_bidir_fwd_ckpt), for
    ssm_scan_bidir_bwd(..., ckpt=ckpt)."""
    _, (Bs, L, ED, N) = _scan_args("ssm_scan_bidir_fwd", x, delta, A, B, C, D, h0, dt_bias, dt_limit, z,
                                   workspace, [("g0", g0, "state"), ("y", y, "seq"), ("h_last", h_last, "state"),
                                               ("g_first", g_first, "state"), ("ckpt", ckpt, "ckpt")])
    dt = _dtype_code(x)
    if y is None:
        import torch
        y = torch.empty_like(x)
    workspace, ws_bytes = _workspace(workspace, ssm_scan_workspace_bytes(Bs, L, ED, N, dt, True), x.device)
    opts = _options(dt_bias, dt_softplus, dt_limit, z)
    head = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(g0), _byref(opts), _ptr(y),
            _ptr(h_last), _ptr(g_first))
    tail = (Bs, L, ED, N, dt, _ptr(workspace), ws_bytes, _stream(x, stream))
    if ckpt is None:
        rc = lib().ssm_scan_bidir_fwd(*head, *tail)
    else:
        rc = lib().ssm_scan_bidir_fwd_ckpt(*head, _ptr(ckpt), ckpt.numel() * 4, *tail)
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_scan_bidir_fwd_ckpt" if ckpt is not None else "ssm_scan_bidir_fwd")
    return y


def ssm_scan_bwd_workspace_bytes(Bs, L, ED, N, dtype=SSM_F32, gate=False):
    return int(lib().ssm_scan_bwd_workspace_bytes(Bs, L, ED, N, int(dtype), int(bool(gate))))


def ssm_scan_bidir_bwd_workspace_bytes(Bs, L, ED, N, dtype=SSM_F32, gate=False):
    return int(lib().ssm_scan_bidir_bwd_workspace_bytes(Bs, L, ED, N, int(dtype), int(bool(gate))))


def _bwd(bidir, x, delta, A, B, C, D, dy, h0, want_dD, want_dh0, out, workspace, stream, dt_bias, dt_softplus,
         dt_limit, want_ddt_bias, z, dh_last=None, g0=None, dg_first=None, want_dg0=False, ckpt=None):
    import torch
    where = "ssm_scan_bidir_bwd" if bidir else "ssm_scan_bwd"
    o = dict(out or {})
    known = {"dx": "seq", "ddelta": "seq", "dA": "a", "dB": "bc", "dC": "bc", "dD": "ed", "dh0": "state",
             "ddt_bias": "ed", "dz": "seq"}
    if bidir:
        known["dg0"] = "state"
    for k in o:
        if k not in known:
            raise ValueError("%s: unknown output %r" % (where, k))
    a, (Bs, L, ED, N) = _scan_args(where, x, delta, A, B, C, D, h0, dt_bias, dt_limit, z, workspace,
                                   [("dy", dy, "seq", True), ("dh_last", dh_last, "state"), ("g0", g0, "state"),
                                    ("dg_first", dg_first, "state"), ("ckpt", ckpt, "ckpt")] +
                                   [(k, v, known[k]) for k, v in o.items()])
    if not bidir and (g0 is not None or dg_first is not None):
        raise ValueError("%s: g0 and dg_first belong to the bidirectional scan" % where)
    dt = _dtype_code(x)
    o.setdefault("dx", torch.empty_like(x))
    o.setdefault("ddelta", torch.empty_like(x))
    o.setdefault("dA", torch.empty((ED, N), dtype=torch.float32, device=x.device))
    o.setdefault("dB", torch.empty_like(B))
    o.setdefault("dC", torch.empty_like(C))
    if want_dD:
        o.setdefault("dD", torch.empty((ED,), dtype=torch.float32, device=x.device))
    if want_dh0:
        o.setdefault("dh0", torch.empty((Bs, ED, N), dtype=torch.float32, device=x.device))
    if bidir and want_dg0:
        o.setdefault("dg0", torch.empty((Bs, ED, N), dtype=torch.float32, device=x.device))
    if want_ddt_bias or dt_bias is not None:
        o.setdefault("ddt_bias", torch.empty((ED,), dtype=torch.float32, device=x.device))
    if z is not None:
        o.setdefault("dz", torch.empty_like(x))
    opts = _options(dt_bias, dt_softplus, dt_limit, z)
    need = (ssm_scan_bidir_bwd_workspace_bytes if bidir else ssm_scan_bwd_workspace_bytes)(Bs, L, ED, N, dt,
                                                                                            z is not None)
    workspace, ws_bytes = _workspace(workspace, need, x.device)
    grads = (_ptr(o["dx"]), _ptr(o["ddelta"]), _ptr(o["dA"]), _ptr(o["dB"]), _ptr(o["dC"]), _ptr(o.get("dD")),
             _ptr(o.get("dh0")))
    tail = (_ptr(o.get("ddt_bias")), _ptr(o.get("dz")), Bs, L, ED, N, dt, _ptr(workspace), ws_bytes,
            _stream(x, stream))
    if bidir and ckpt is not None:
        where = "ssm_scan_bidir_bwd_ckpt"
        rc = lib().ssm_scan_bidir_bwd_ckpt(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                                           _ptr(g0), _byref(opts), _ptr(dy), _ptr(dh_last), _ptr(dg_first),
                                           _ptr(ckpt), ckpt.numel() * 4, *grads, _ptr(o.get("dg0")), *tail)
    elif bidir:
        rc = lib().ssm_scan_bidir_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(g0),
                                      _byref(opts), _ptr(dy), _ptr(dh_last), _ptr(dg_first), *grads,
                                      _ptr(o.get("dg0")), *tail)
    elif ckpt is not None:
        where = "ssm_scan_bwd_ckpt"
        rc = lib().ssm_scan_bwd_ckpt(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                                     _byref(opts), _ptr(dy), _ptr(dh_last), _ptr(ckpt), ckpt.numel() * 4, *grads,
                                     *tail)
    else:
        rc = lib().ssm_scan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _byref(opts),
                                _ptr(dy), _ptr(dh_last), *grads, *tail)
    if rc != SSM_OK:
        raise SSMError(rc, where)
    return o


def ssm_scan_bwd(x, delta, A, B, C, D, dy, h0=None, want_dD=True, want_dh0=False, out=None, workspace=None,
                 stream=None, dt_bias=None, dt_softplus=False, dt_limit=None, want_ddt_bias=False, z=None,
                 dh_last=None, ckpt=None):
    """Gradients of sum(dy * y) (+ sum(dh_last * h_last) when dh_last, the
    final state's gradient, is given) for y = ssm_scan_fwd(x, delta, A, B,
    C, D, h0=h0, dt_bias=dt_bias, dt_softplus=dt_softplus, dt_limit=dt_limit,
    z=z).

    Returns a dict with dx, ddelta (like x; the raw delta's gradient), dA
    (like A), dB, dC (like B), dD (ED,) float32 if want_dD, dh0 (Bs, ED, N)
    float32 if want_dh0, ddt_bias (ED,) float32 if dt_bias is given or
    want_ddt_bias, dz (like x) if z is given. Tensors given in ``out`` (same
    keys) are written instead of new ones. ckpt: the round checkpoints that
    ssm_scan_fwd(..., ckpt=ckpt) wrote for the same inputs (the backward
    then skips its own forward sweep; ssm_scan_bwd_ckpt).
    """
    return _bwd(False, x, delta, A, B, C, D, dy, h0, want_dD, want_dh0, out, workspace, stream, dt_bias,
                dt_softplus, dt_limit, want_ddt_bias, z, dh_last=dh_last, ckpt=ckpt)


def ssm_scan_bidir_bwd(x, delta, A, B, C, D, dy, h0=None, want_dD=True, want_dh0=False, out=None, workspace=None,
                       stream=None, dt_bias=None, dt_softplus=False, dt_limit=None, want_ddt_bias=False, z=None,
                       g0=None, dh_last=None, dg_first=None, want_dg0=False, ckpt=None):
    """Gradients of sum(dy * y) (+ sum(dh_last * h_last) + sum(dg_first *
    g_first) for the final states' gradients when given) for y =
    ssm_scan_bidir_fwd(x, delta, A, B, C, D, h0=h0, g0=g0, <step-size
    options>, z=z), with the outputs of ssm_scan_bwd and dg0 (the gradient of
    g0) if want_dg0. ckpt: the forward direction's round checkpoints that
    ssm_scan_bidir_fwd(..., ckpt=ckpt) wrote for the same inputs
    (ssm_scan_bidir_bwd_ckpt)."""
    return _bwd(True, x, delta, A, B, C, D, dy, h0, want_dD, want_dh0, out, workspace, stream, dt_bias,
                dt_softplus, dt_limit, want_ddt_bias, z, dh_last=dh_last, g0=g0, dg_first=dg_first,
                want_dg0=want_dg0, ckpt=ckpt)


def _ssd_args(where, x, dt, A, B, C, D, h0, dt_bias, dt_limit, z, workspace, outs):
    """Validates the multi-head scan's arguments; returns (Bs, L, H, P, G, N)."""
    import torch
    a = _Args(where, x, 4)
    Bs, L, H, P = (int(v) for v in x.shape)
    f32 = torch.float32
    if not isinstance(B, torch.Tensor) or B.dim() != 4:
        raise ValueError("%s: B must be a 4-D tensor (Bs, L, G, N)" % where)
    G, N = int(B.shape[2]), int(B.shape[3])
    a.check("dt", dt, (Bs, L, H), required=True)
    a.check("A", A, (H,), f32, required=True)
    a.check("B", B, (Bs, L, G, N), required=True)
    a.check("C", C, (Bs, L, G, N), required=True)
    a.check("D", D, (H,), f32)
    a.check("h0", h0, (Bs, H, P, N), f32)
    a.check("dt_bias", dt_bias, (H,), f32)
    a.check("z", z, (Bs, L, H, P))
    a.limit(dt_limit)
    for name, t, kind in outs:
        if kind == "seq":
            a.check(name, t, (Bs, L, H, P))
        else:
            a.check(name, t, (Bs, H, P, N), f32)
    a.workspace(workspace)
    a.check_gpu()
    return Bs, L, H, P, G, N


def ssm_ssd_workspace_bytes(Bs, L, H, P, dtype=SSM_F32):
    """Workspace bytes of ssm_ssd_fwd on the current device (nonzero when the
    sequences are split into ranges: fewer (batch row, head) pairs than
    compute units)."""
    return lib().ssm_ssd_workspace_bytes(Bs, L, H, P, dtype)


def ssm_ssd_fwd(x, dt, A, B, C, D=None, y=None, h_last=None, h0=None, stream=None, dt_bias=None,
                dt_softplus=False, dt_limit=None, z=None, workspace=None):
    """Multi-head selective scan: x (Bs, L, H, P), dt (Bs, L, H), A (H,),
    B and C (Bs, L, G, N), D (H,) or None, h0 (Bs, H, P, N) or None.
    dt_bias (H,) / dt_softplus / dt_limit pre-process dt, z (like x) gates
    the output. Returns y (Bs, L, H, P); the final state goes to h_last if
    given. A workspace (uint8, ssm_ssd_workspace_bytes) is allocated when
    needed and not given."""
    import torch
    Bs, L, H, P, G, N = _ssd_args("ssm_ssd_fwd", x, dt, A, B, C, D, h0, dt_bias, dt_limit, z, workspace,
                                  [("y", y, "seq"), ("h_last", h_last, "state")])
    dtc = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    workspace, wsb = _workspace(workspace, lib().ssm_ssd_workspace_bytes(Bs, L, H, P, dtc), x.device)
    opts = _options(dt_bias, dt_softplus, dt_limit, z)
    rc = lib().ssm_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _byref(opts), _ptr(y),
                           _ptr(h_last), Bs, L, H, P, G, N, dtc, _ptr(workspace), wsb, _stream(x, stream))
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_ssd_fwd")
    return y


def ssm_ssd_bidir_workspace_bytes(Bs, L, H, P, dtype=SSM_F32):
    """Workspace bytes of ssm_ssd_bidir_fwd on the current device (SSM_BF16:
    the reverse sweep's float32 partial output; a split sequence: both
    sweeps' range states)."""
    return lib().ssm_ssd_bidir_workspace_bytes(Bs, L, H, P, dtype)


def ssm_ssd_bidir_fwd(x, dt, A, B, C, D=None, y=None, h_last=None, g_first=None, h0=None, workspace=None,
                      stream=None, dt_bias=None, dt_softplus=False, dt_limit=None, z=None, g0=None):
    """Bidirectional multi-head scan: ssm_ssd_fwd plus the same scan in
    decreasing time from g0 (zero if None; no D), with the options of
    ssm_ssd_fwd (the gate applies to the sum). Returns y; the final states
    go to h_last (forward) and g_first (reverse) if given."""
    import torch
    Bs, L, H, P, G, N = _ssd_args("ssm_ssd_bidir_fwd", x, dt, A, B, C, D, h0, dt_bias, dt_limit, z, workspace,
                                  [("g0", g0, "state"), ("y", y, "seq"), ("h_last", h_last, "state"),
                                   ("g_first", g_first, "state")])
    dtc = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    workspace, wsb = _workspace(workspace, lib().ssm_ssd_bidir_workspace_bytes(Bs, L, H, P, dtc), x.device)
    opts = _options(dt_bias, dt_softplus, dt_limit, z)
    rc = lib().ssm_ssd_bidir_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(g0),
                                 _byref(opts),
                                 _ptr(y), _ptr(h_last), _ptr(g_first), Bs, L, H, P, G, N, dtc, _ptr(workspace), wsb,
                                 _stream(x, stream))
    if rc != SSM_OK:
        raise SSMError(rc, "ssm_ssd_bidir_fwd")
    return y

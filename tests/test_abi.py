"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import state_space_model_selective_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

# fake device addresses, 16-byte aligned and far apart; only used on paths that
# must fail validation before anything touches them. Where a GPU is present a
# validation gap would launch a kernel on them, so these host-only checks are
# skipped there (the GPU tests load and call the same library).
P = [0x10000000 * (i + 1) for i in range(26)]

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="calls the library with fake device addresses: host-only")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"ssm_scan_fwd", "ssm_scan_bidir_fwd", "ssm_scan_workspace_bytes", "ssm_status_str"} <= set(names)
    lib = ctypes.CDLL(ssm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(9):
        assert ssm.status_str(s) != "unknown status"
    assert ssm.status_str(999) == "unknown status"


def fwd(**kw):
    args = dict(x=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=P[5], y=P[6], h=P[7], h0=P[10], opts=None, Bs=2,
                L=64, ED=64, N=16, dtype=ssm.SSM_F32, ws=None, ws_bytes=0)
    args.update(kw)
    return ssm.lib().ssm_scan_fwd(args["x"], args["delta"], args["A"], args["B"], args["C"], args["D"], args["h0"],
                                  args["opts"], args["y"],
                                  args["h"], args["Bs"], args["L"], args["ED"], args["N"], args["dtype"], args["ws"],
                                  args["ws_bytes"], None)


def bidir(**kw):
    args = dict(x=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=P[5], y=P[6], h=P[7], g=P[8], h0=P[10], g0=P[15],
                opts=None, Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_F32, ws=None, ws_bytes=0)
    args.update(kw)
    return ssm.lib().ssm_scan_bidir_fwd(args["x"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                        args["h0"], args["g0"], args["opts"], args["y"], args["h"], args["g"],
                                        args["Bs"], args["L"], args["ED"], args["N"], args["dtype"], args["ws"],
                                        args["ws_bytes"], None)


def test_reverse_initial_state_arguments():
    assert bidir(g0=P[15] + 4) == ssm.SSM_ERR_UNSUPPORTED     # misaligned
    assert bidir(g=P[15]) == ssm.SSM_ERR_ALIAS                # g_first on top of g0
    assert bidir(y=P[15] - 64) == ssm.SSM_ERR_ALIAS           # y running into g0
    none = dict(x=None, delta=None, B=None, C=None, D=None, y=None, h=None, g=None, h0=None, g0=None)
    assert bidir(**dict(none, Bs=0, ED=0)) == ssm.SSM_OK


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "y"])
def test_null_pointer(name):
    assert fwd(**{name: None}) == ssm.SSM_ERR_NULL
    assert bidir(**{name: None}) == ssm.SSM_ERR_NULL


@pytest.mark.parametrize("dim,val", [("Bs", -1), ("L", -1), ("ED", -1), ("N", 0), ("N", -1)])
def test_bad_dimension(dim, val):
    assert fwd(**{dim: val}) == ssm.SSM_ERR_DIM
    assert bidir(**{dim: val}) == ssm.SSM_ERR_DIM


# Empty inputs are valid. The calls below have nothing to write (no final
# state requested, or no channels), so they return before any HIP call, and
# every buffer without elements may be NULL. (Empty calls that do write --
# h_last = h0, zero gradients -- are GPU tests.)
E_NULL = dict(x=None, delta=None, B=None, C=None, D=None, y=None, h=None, h0=None)


# (with ED = 0, B and C -- (Bs, L, N) -- still have elements and stay given)
@pytest.mark.parametrize("sizes", [dict(Bs=0), dict(ED=0, A=None, B=P[3], C=P[4]), dict(Bs=0, L=0, ED=0, A=None)])
def test_empty_inputs_are_valid(sizes):
    assert fwd(**dict(E_NULL, **sizes)) == ssm.SSM_OK
    assert bidir(**dict(E_NULL, g=None, **sizes)) == ssm.SSM_OK
    for bi in (0, 1):
        assert ssm.ssm_scan_workspace_bytes(sizes.get("Bs", 2), sizes.get("L", 64), sizes.get("ED", 64), 16,
                                            ssm.SSM_BF16, bi) == 0


def test_empty_sequence_without_states_is_valid():
    # L = 0 with A given: no output, nothing requested
    assert fwd(**dict(E_NULL, L=0)) == ssm.SSM_OK
    assert bidir(**dict(E_NULL, L=0, g=None)) == ssm.SSM_OK


def test_size_overflow():
    assert fwd(Bs=1 << 40, L=1 << 20, ED=1 << 10) == ssm.SSM_ERR_DIM


@pytest.mark.parametrize("N", [1, 8, 15, 17, 32])
def test_unsupported_state_size(N):
    assert fwd(N=N) == ssm.SSM_ERR_UNSUPPORTED


def test_unknown_dtype():
    assert fwd(dtype=7) == ssm.SSM_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "y", "h", "h0"])
def test_misaligned_pointer(name):
    base = dict(x=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=P[5], y=P[6], h=P[7], h0=P[10])
    assert fwd(**{name: base[name] + 4}) == ssm.SSM_ERR_UNSUPPORTED


def test_output_aliasing_an_input():
    assert fwd(y=P[0]) == ssm.SSM_ERR_ALIAS            # y on top of x
    assert fwd(y=P[1] + 4096) == ssm.SSM_ERR_ALIAS     # y inside delta
    assert fwd(h=P[6] + 64) == ssm.SSM_ERR_ALIAS       # h_last inside y
    assert bidir(g=P[7]) == ssm.SSM_ERR_ALIAS          # g_first on h_last
    assert fwd(h=P[10]) == ssm.SSM_ERR_ALIAS           # h_last on top of h0


def test_workspace_query_and_check():
    assert ssm.ssm_scan_workspace_bytes(2, 64, 64, 16, ssm.SSM_F32, False) == 0
    assert ssm.ssm_scan_workspace_bytes(0, 64, 64, 16, ssm.SSM_F32, False) == 0
    need = ssm.ssm_scan_workspace_bytes(2, 64, 64, 16, ssm.SSM_BF16, True)
    if need:
        assert bidir(dtype=ssm.SSM_BF16) == ssm.SSM_ERR_WORKSPACE
        assert bidir(dtype=ssm.SSM_BF16, ws=P[9], ws_bytes=need - 1) == ssm.SSM_ERR_WORKSPACE
        assert bidir(dtype=ssm.SSM_BF16, ws=P[6], ws_bytes=need) == ssm.SSM_ERR_ALIAS


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 16)
    with pytest.raises(RuntimeError):
        ssm.ssm_scan_fwd(x, x, torch.zeros(16, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 16))


def opts(**kw):
    o = ssm.SSMOptions(None, 0, -float("inf"), float("inf"), None)
    for k, v in kw.items():
        setattr(o, k, v)
    return ctypes.byref(o), o


def test_options_validation():
    ref, _ = opts(dt_min=0.5, dt_max=0.1)
    assert fwd(opts=ref) == ssm.SSM_ERR_ARG
    ref, _ = opts(dt_min=float("nan"))
    assert bidir(opts=ref) == ssm.SSM_ERR_ARG
    ref, _ = opts(z=P[6])                               # gate on top of y
    assert fwd(opts=ref) == ssm.SSM_ERR_ALIAS
    ref, _ = opts(dt_bias=P[11] + 8)                    # misaligned bias
    assert fwd(opts=ref) == ssm.SSM_ERR_UNSUPPORTED
    ref, _ = opts(z=P[11] + 4)
    assert fwd(opts=ref) == ssm.SSM_ERR_UNSUPPORTED
    ref, _ = opts(dt_bias=P[7])                         # h_last on top of the bias
    assert fwd(opts=ref) == ssm.SSM_ERR_ALIAS


BWD_PTRS = ["x", "delta", "A", "B", "C", "D", "h0", "opts", "dy", "dx", "ddelta", "dA", "dB", "dC", "dD", "dh0",
            "ddt_bias", "dz", "ws", "dh_last", "g0", "dg_first", "dg0"]
BWD_DEFAULT = {n: P[i] for i, n in enumerate(BWD_PTRS)}  # the default pointer of each argument
# argument order of the two entry points
BWD_ORDER = ["x", "delta", "A", "B", "C", "D", "h0", "opts", "dy", "dh_last", "dx", "ddelta", "dA", "dB", "dC", "dD",
             "dh0", "ddt_bias", "dz"]
BIDIR_BWD_ORDER = ["x", "delta", "A", "B", "C", "D", "h0", "g0", "opts", "dy", "dh_last", "dg_first", "dx", "ddelta",
                   "dA", "dB", "dC", "dD", "dh0", "dg0", "ddt_bias", "dz"]


def bwd(**kw):
    args = dict(BWD_DEFAULT)
    args.update(opts=None, Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_F32)  # (opts is read on the host)
    args["ws_bytes"] = ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_F32)
    args.update(kw)
    return ssm.lib().ssm_scan_bwd(*[args[n] for n in BWD_ORDER], args["Bs"], args["L"], args["ED"], args["N"],
                                  args["dtype"], args["ws"], args["ws_bytes"], None)


def test_bwd_workspace_size():
    need = ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_F32)
    # checkpoints (2 rows x 2 rounds x 64 channels x 16 states), dB and dC
    # partials (4 groups x 2 x 64 x 16 each), dA and dD partials, all float32
    assert need >= 4 * (2 * 2 * 64 * 16 + 2 * 4 * 2 * 64 * 16 + 2 * 64 * 17)
    assert ssm.ssm_scan_bwd_workspace_bytes(0, 64, 64, 16, ssm.SSM_F32) == 0
    assert ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 8, ssm.SSM_F32) == 0


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "dy", "dx", "ddelta", "dA", "dB", "dC"])
def test_bwd_null_pointer(name):
    assert bwd(**{name: None}) == ssm.SSM_ERR_NULL


def test_bwd_optional_pointers_may_be_null():
    # D, h0, dD, dh0 are optional: with them NULL the call gets past the NULL
    # check and fails only on the fake (misaligned) workspace below
    assert bwd(D=None, h0=None, dD=None, dh0=None, ws=P[18] + 4) == ssm.SSM_ERR_UNSUPPORTED


def test_bwd_empty_inputs_are_valid():
    # no batch rows and no channels: no gradient has an element
    none = {n: None for n in BWD_PTRS}
    assert bwd(**dict(none, Bs=0, ED=0, ws_bytes=0)) == ssm.SSM_OK
    assert ssm.ssm_scan_bwd_workspace_bytes(2, 0, 64, 16, ssm.SSM_F32) == 0
    assert ssm.ssm_scan_bwd_workspace_bytes(2, 64, 0, 16, ssm.SSM_BF16) == 0


def test_bwd_validation():
    assert bwd(L=-1) == ssm.SSM_ERR_DIM
    assert bwd(N=8) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(dtype=3) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(dB=P[12] + 4) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(ws=None) == ssm.SSM_ERR_WORKSPACE
    assert bwd(ws_bytes=1024) == ssm.SSM_ERR_WORKSPACE
    assert bwd(dx=P[0]) == ssm.SSM_ERR_ALIAS              # dx on top of x
    assert bwd(ddelta=P[9] + 256) == ssm.SSM_ERR_ALIAS    # ddelta inside dx
    assert bwd(dh0=P[6]) == ssm.SSM_ERR_ALIAS             # dh0 on top of h0
    assert bwd(ws=P[8]) == ssm.SSM_ERR_ALIAS              # workspace on top of dy
    assert bwd(dh_last=P[19] + 8) == ssm.SSM_ERR_UNSUPPORTED   # misaligned final-state gradient
    assert bwd(dh0=P[19]) == ssm.SSM_ERR_ALIAS            # dh0 on top of dh_last
    assert bwd(dh_last=P[9]) == ssm.SSM_ERR_ALIAS         # dx on top of dh_last


SSD_PTRS = ["x", "dt", "A", "B", "C", "D", "h0", "opts", "y", "h"]


SP = {n: P[i] for i, n in enumerate(SSD_PTRS)}  # the default pointer of each argument


def ssd(**kw):
    args = dict(SP)
    args.update(opts=None, Bs=2, L=64, H=4, P=64, G=1, N=128, dtype=ssm.SSM_F32)
    args.update(kw)
    return ssm.lib().ssm_ssd_fwd(*[args[n] for n in SSD_PTRS], args["Bs"], args["L"], args["H"], args["P"],
                                 args["G"], args["N"], args["dtype"], args.get("ws"), args.get("ws_bytes", 0), None)


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "y"])
def test_ssd_null_pointer(name):
    assert ssd(**{name: None}) == ssm.SSM_ERR_NULL


def test_ssd_empty_inputs_are_valid():
    none = dict(x=None, dt=None, B=None, C=None, D=None, h0=None, y=None, h=None)
    assert ssd(**dict(none, L=0)) == ssm.SSM_OK
    assert ssd(**dict(none, Bs=0)) == ssm.SSM_OK
    assert ssd(**dict(none, L=0, A=None)) == ssm.SSM_ERR_NULL   # A (H) is never empty
    assert ssd_bidir(**dict(none, g=None, g0=None, ws=None, ws_bytes=0, L=0)) == ssm.SSM_OK


def test_ssd_validation():
    assert ssd(L=-1) == ssm.SSM_ERR_DIM
    assert ssd(H=0) == ssm.SSM_ERR_DIM
    assert ssd(H=3, G=2) == ssm.SSM_ERR_DIM          # heads not a multiple of groups
    assert ssd(P=32) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(N=16) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(dtype=5) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(dt=SP["dt"] + 8) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd(y=SP["x"] + 64) == ssm.SSM_ERR_ALIAS   # y inside x
    assert ssd(h=SP["y"]) == ssm.SSM_ERR_ALIAS        # h_last on top of y
    assert ssd(h=SP["h0"]) == ssm.SSM_ERR_ALIAS       # h_last on top of h0


SSD_BI_PTRS = ["x", "dt", "A", "B", "C", "D", "h0", "opts", "y", "h", "g"]
SSD_BI_ORDER = ["x", "dt", "A", "B", "C", "D", "h0", "g0", "opts", "y", "h", "g"]


BP = dict({n: P[i] for i, n in enumerate(SSD_BI_PTRS)}, ws=P[12], g0=P[24])  # default pointers


def ssd_bidir(**kw):
    args = dict(BP)
    args.update(opts=None, Bs=2, L=64, H=4, P=64, G=1, N=128, dtype=ssm.SSM_BF16)
    args["ws_bytes"] = ssm.ssm_ssd_bidir_workspace_bytes(2, 64, 4, 64, ssm.SSM_BF16)
    args.update(kw)
    return ssm.lib().ssm_ssd_bidir_fwd(*[args[n] for n in SSD_BI_ORDER], args["Bs"], args["L"], args["H"], args["P"],
                                       args["G"], args["N"], args["dtype"], args["ws"], args["ws_bytes"], None)


def test_ssd_bidir_workspace_size():
    # the reverse sweep's float32 partial output, one value per element of y
    # (no device here: no split plan, so nothing else)
    assert ssm.ssm_ssd_bidir_workspace_bytes(2, 64, 4, 64, ssm.SSM_BF16) >= 4 * 2 * 64 * 4 * 64
    assert ssm.ssm_ssd_bidir_workspace_bytes(2, 64, 4, 64, ssm.SSM_F32) == 0
    assert ssm.ssm_ssd_bidir_workspace_bytes(0, 64, 4, 64, ssm.SSM_BF16) == 0
    assert ssm.ssm_ssd_workspace_bytes(2, 64, 4, 64, ssm.SSM_F32) == 0
    assert ssm.ssm_ssd_workspace_bytes(2, 64, 4, 64, ssm.SSM_BF16) == 0


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "y"])
def test_ssd_bidir_null_pointer(name):
    assert ssd_bidir(**{name: None}) == ssm.SSM_ERR_NULL


def test_ssd_bidir_validation():
    need = ssm.ssm_ssd_bidir_workspace_bytes(2, 64, 4, 64, ssm.SSM_BF16)
    assert ssd_bidir(L=-1) == ssm.SSM_ERR_DIM
    assert ssd_bidir(N=96) == ssm.SSM_ERR_UNSUPPORTED
    assert ssd_bidir(ws=None) == ssm.SSM_ERR_WORKSPACE
    assert ssd_bidir(ws_bytes=need - 1) == ssm.SSM_ERR_WORKSPACE
    assert ssd_bidir(ws=BP["ws"] + 4) == ssm.SSM_ERR_WORKSPACE     # misaligned workspace
    assert ssd_bidir(g=BP["h"]) == ssm.SSM_ERR_ALIAS               # g_first on top of h_last
    assert ssd_bidir(g=BP["y"] + 64) == ssm.SSM_ERR_ALIAS          # g_first inside y
    assert ssd_bidir(ws=BP["y"]) == ssm.SSM_ERR_ALIAS              # workspace on top of y
    assert ssd_bidir(ws=BP["x"]) == ssm.SSM_ERR_ALIAS              # workspace on top of x
    assert ssd_bidir(g0=BP["g0"] + 4) == ssm.SSM_ERR_UNSUPPORTED   # misaligned reverse initial state
    assert ssd_bidir(g=BP["g0"]) == ssm.SSM_ERR_ALIAS              # g_first on top of g0
    assert ssd_bidir(ws=BP["g0"]) == ssm.SSM_ERR_ALIAS             # workspace on top of g0
    # float32 needs no workspace: the reverse partial is kept in y itself
    assert ssd_bidir(dtype=ssm.SSM_F32, ws=None, ws_bytes=0, N=96) == ssm.SSM_ERR_UNSUPPORTED


def test_ssd_options_validation():
    ref, _ = opts(dt_min=0.5, dt_max=0.1)
    assert ssd(opts=ref) == ssm.SSM_ERR_ARG
    ref, _ = opts(dt_max=float("nan"))
    assert ssd_bidir(opts=ref) == ssm.SSM_ERR_ARG
    ref, _ = opts(z=SP["y"])                            # gate on top of y
    assert ssd(opts=ref) == ssm.SSM_ERR_ALIAS
    ref, _ = opts(dt_bias=SP["h"])                      # h_last on top of the bias
    assert ssd(opts=ref) == ssm.SSM_ERR_ALIAS
    ref, _ = opts(z=P[13] + 8)                          # misaligned gate
    assert ssd(opts=ref) == ssm.SSM_ERR_UNSUPPORTED
    ref, _ = opts(dt_bias=P[13] + 4)                    # misaligned bias
    assert ssd_bidir(opts=ref) == ssm.SSM_ERR_UNSUPPORTED
    ref, _ = opts(z=BP["ws"])                           # gate inside the bidirectional workspace
    assert ssd_bidir(opts=ref) == ssm.SSM_ERR_ALIAS
    # valid options get past validation to the (missing) workspace check
    ref, _ = opts(dt_bias=P[13], dt_softplus=1, dt_min=0.0, dt_max=1.0, z=P[14])
    assert ssd_bidir(opts=ref, ws=None) == ssm.SSM_ERR_WORKSPACE


def bidir_bwd(**kw):
    args = dict(BWD_DEFAULT)
    args.update(opts=None, Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_BF16)
    args["ws_bytes"] = ssm.ssm_scan_bidir_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_BF16)
    args.update(kw)
    return ssm.lib().ssm_scan_bidir_bwd(*[args[n] for n in BIDIR_BWD_ORDER], args["Bs"], args["L"], args["ED"],
                                        args["N"], args["dtype"], args["ws"], args["ws_bytes"], None)


def test_bidir_bwd_workspace_size():
    plain = ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_BF16)
    both = ssm.ssm_scan_bidir_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_BF16)
    # both directions' dB / dC partials (4 groups x 2 x 64 x 16 each, twice)
    # and the forward direction's float32 dx and ddelta
    assert both >= plain + 4 * (2 * 4 * 2 * 64 * 16 + 2 * 2 * 64 * 64)
    assert ssm.ssm_scan_bidir_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_F32) < both
    assert ssm.ssm_scan_bidir_bwd_workspace_bytes(0, 64, 64, 16, ssm.SSM_BF16) == 0


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "dy", "dx", "ddelta", "dA", "dB", "dC"])
def test_bidir_bwd_null_pointer(name):
    assert bidir_bwd(**{name: None}) == ssm.SSM_ERR_NULL


def test_bidir_bwd_validation():
    plain = ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_BF16)
    assert bidir_bwd(L=-1) == ssm.SSM_ERR_DIM
    assert bidir_bwd(N=8) == ssm.SSM_ERR_UNSUPPORTED
    assert bidir_bwd(ws=None) == ssm.SSM_ERR_WORKSPACE
    assert bidir_bwd(ws_bytes=plain) == ssm.SSM_ERR_WORKSPACE   # the one-direction size is too small
    assert bidir_bwd(dx=P[0]) == ssm.SSM_ERR_ALIAS
    assert bidir_bwd(dg0=P[20]) == ssm.SSM_ERR_ALIAS          # dg0 on top of g0
    assert bidir_bwd(dg0=P[21]) == ssm.SSM_ERR_ALIAS          # dg0 on top of dg_first
    assert bidir_bwd(dh0=P[22]) == ssm.SSM_ERR_ALIAS          # dh0 on top of dg0
    assert bidir_bwd(g0=P[20] + 4) == ssm.SSM_ERR_UNSUPPORTED
    assert bidir_bwd(dg_first=P[21] + 8) == ssm.SSM_ERR_UNSUPPORTED
    none = {n: None for n in BWD_PTRS}
    assert bidir_bwd(**dict(none, Bs=0, ED=0, ws_bytes=0)) == ssm.SSM_OK


def test_bwd_options_validation():
    gated = ssm.SSMOptions(None, 1, -float("inf"), float("inf"), P[19])
    assert bwd(opts=ctypes.byref(gated), dz=None) == ssm.SSM_ERR_NULL            # the gate needs dz
    assert bidir_bwd(opts=ctypes.byref(gated), dz=None) == ssm.SSM_ERR_NULL
    assert bwd(opts=ctypes.byref(gated)) == ssm.SSM_ERR_WORKSPACE                # and the larger workspace
    assert bidir_bwd(opts=ctypes.byref(gated)) == ssm.SSM_ERR_WORKSPACE
    need = ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_F32, gate=True)
    assert bwd(opts=ctypes.byref(gated), ws_bytes=need, dz=P[0]) == ssm.SSM_ERR_ALIAS   # dz on top of x
    assert bwd(opts=ctypes.byref(gated), ws_bytes=need, dz=P[17] + 4) == ssm.SSM_ERR_UNSUPPORTED
    inverted = ssm.SSMOptions(None, 0, 0.5, 0.1, None)
    assert bwd(opts=ctypes.byref(inverted)) == ssm.SSM_ERR_ARG
    nan = ssm.SSMOptions(None, 0, float("nan"), 1.0, None)
    assert bidir_bwd(opts=ctypes.byref(nan)) == ssm.SSM_ERR_ARG
    misaligned = ssm.SSMOptions(P[19] + 4, 1, 0.0, 1.0, None)
    assert bwd(opts=ctypes.byref(misaligned)) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(ddt_bias=P[0]) == ssm.SSM_ERR_ALIAS                           # ddt_bias on top of x


@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("dtype", [ssm.SSM_F32, ssm.SSM_BF16])
def test_gated_backward_workspace(bidir, dtype):
    """With the gate the workspace also holds dy silu(z): one float32 value
    per element of x, after the backward's own area."""
    q = ssm.ssm_scan_bidir_bwd_workspace_bytes if bidir else ssm.ssm_scan_bwd_workspace_bytes
    plain, gated = q(2, 300, 64, 16, dtype), q(2, 300, 64, 16, dtype, gate=True)
    assert gated >= plain + 2 * 300 * 64 * 4
    assert gated < plain + 2 * 300 * 64 * 4 + 1024
    assert q(0, 300, 64, 16, dtype, gate=True) == 0


def test_one_hip_runtime_whatever_the_call_order():
    # The library is loaded with torch's HIP runtime already in the process,
    # so that both use one runtime: a library call made before any torch call
    # must not bring in a second (torch would then find no device).
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import state_space_model_selective_amd as ssm\n"
            "ssm.ssm_scan_workspace_bytes(1, 64, 64, 16)\n"
            "import torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps))\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def fwd_ckpt(**kw):
    args = dict(x=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=P[5], y=P[6], h=P[7], h0=P[10], ck=P[20], opts=None,
                Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_F32, ws=None, ws_bytes=0)
    args["ck_bytes"] = ssm.lib().ssm_scan_ckpt_bytes(2, 64, 64, 16)
    args.update(kw)
    return ssm.lib().ssm_scan_fwd_ckpt(args["x"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                       args["h0"], args["opts"], args["y"], args["h"], args["ck"], args["ck_bytes"],
                                       args["Bs"], args["L"], args["ED"], args["N"], args["dtype"], args["ws"],
                                       args["ws_bytes"], None)


def test_checkpoint_bytes():
    q = ssm.lib().ssm_scan_ckpt_bytes
    # (Bs, ceil(L / 32), 16 ceil(ED / 16), 16) float32
    assert q(2, 64, 64, 16) == 2 * 2 * 64 * 16 * 4
    assert q(3, 65, 20, 16) == 3 * 3 * 32 * 16 * 4
    assert q(1, 1, 1, 16) == 16 * 16 * 4
    assert q(2, 0, 64, 16) == 0 and q(0, 64, 64, 16) == 0
    assert q(2, 64, 64, 8) == 0                     # N other than 16
    assert q(1, 1 << 62, 1 << 20, 16) == 0          # overflow
    assert ssm.ssm_scan_ckpt_shape(3, 65, 20) == (3, 3, 32, 16)


def test_forward_checkpoint_validation():
    assert fwd_ckpt(ck=None) == ssm.SSM_ERR_NULL
    assert fwd_ckpt(ck=P[20] + 8) == ssm.SSM_ERR_UNSUPPORTED       # misaligned
    assert fwd_ckpt(ck_bytes=1024) == ssm.SSM_ERR_WORKSPACE         # too small
    assert fwd_ckpt(ck=P[0]) == ssm.SSM_ERR_ALIAS                   # on top of x
    assert fwd_ckpt(ck=P[6] + 256) == ssm.SSM_ERR_ALIAS             # inside y
    none = dict(x=None, delta=None, B=None, C=None, D=None, y=None, h=None, h0=None, ck=None)
    assert fwd_ckpt(**dict(none, Bs=0, ED=0)) == ssm.SSM_OK         # nothing to scan: no checkpoints


def bwd_ckpt(**kw):
    args = dict(BWD_DEFAULT)
    args.update(opts=None, Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_F32, ck=P[24])
    args["ws_bytes"] = ssm.ssm_scan_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_F32)
    args["ck_bytes"] = ssm.lib().ssm_scan_ckpt_bytes(2, 64, 64, 16)
    args.update(kw)
    head = [args[n] for n in BWD_ORDER[:10]]
    tail = [args[n] for n in BWD_ORDER[10:]]
    return ssm.lib().ssm_scan_bwd_ckpt(*head, args["ck"], args["ck_bytes"], *tail, args["Bs"], args["L"], args["ED"],
                                       args["N"], args["dtype"], args["ws"], args["ws_bytes"], None)


def test_backward_checkpoint_validation():
    assert bwd_ckpt(ck=None) == ssm.SSM_ERR_NULL
    assert bwd_ckpt(ck=P[24] + 4) == ssm.SSM_ERR_UNSUPPORTED       # misaligned
    assert bwd_ckpt(ck_bytes=64) == ssm.SSM_ERR_WORKSPACE          # too small
    assert bwd_ckpt(ck=P[9]) == ssm.SSM_ERR_ALIAS                  # dx on top of the checkpoints
    assert bwd_ckpt(ck=P[18]) == ssm.SSM_ERR_ALIAS                 # the workspace on top of them
    none = {n: None for n in BWD_PTRS}
    assert bwd_ckpt(**dict(none, ck=None, Bs=0, ED=0, ws_bytes=0)) == ssm.SSM_OK


def test_binding_checks_checkpoint_tensors():
    import torch
    x = torch.zeros(2, 40, 20)
    d, B, C = torch.zeros(2, 40, 20), torch.zeros(2, 40, 16), torch.zeros(2, 40, 16)
    A = torch.zeros(20, 16)
    with pytest.raises(ValueError, match="ckpt must have shape"):
        ssm.ssm_scan_fwd(x, d, A, B, C, ckpt=torch.zeros(2, 2, 20, 16))
    with pytest.raises(TypeError, match="ckpt must be torch.float32"):
        ssm.ssm_scan_fwd(x, d, A, B, C, ckpt=torch.zeros(2, 2, 32, 16, dtype=torch.float64))
    with pytest.raises(TypeError):
        ssm.ssm_scan_bwd(x, d, A, B, C, None, x, ckpt=torch.zeros(2, 2, 32, 16, dtype=torch.bfloat16))


def bidir_fwd_ckpt(**kw):
    args = dict(x=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=P[5], y=P[6], h=P[7], g=P[8], h0=P[10], g0=P[15],
                ck=P[20], opts=None, Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_F32, ws=None, ws_bytes=0)
    args["ck_bytes"] = ssm.lib().ssm_scan_ckpt_bytes(2, 64, 64, 16)
    args.update(kw)
    return ssm.lib().ssm_scan_bidir_fwd_ckpt(args["x"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                                             args["h0"], args["g0"], args["opts"], args["y"], args["h"], args["g"],
                                             args["ck"], args["ck_bytes"], args["Bs"], args["L"], args["ED"],
                                             args["N"], args["dtype"], args["ws"], args["ws_bytes"], None)


def test_bidir_forward_checkpoint_validation():
    assert bidir_fwd_ckpt(ck=None) == ssm.SSM_ERR_NULL
    assert bidir_fwd_ckpt(ck=P[20] + 8) == ssm.SSM_ERR_UNSUPPORTED       # misaligned
    assert bidir_fwd_ckpt(ck_bytes=1024) == ssm.SSM_ERR_WORKSPACE         # too small
    assert bidir_fwd_ckpt(ck=P[15]) == ssm.SSM_ERR_ALIAS                  # on top of g0
    assert bidir_fwd_ckpt(ck=P[8] + 256) == ssm.SSM_ERR_ALIAS             # inside g_first
    none = dict(x=None, delta=None, B=None, C=None, D=None, y=None, h=None, g=None, h0=None, g0=None, ck=None)
    assert bidir_fwd_ckpt(**dict(none, Bs=0, ED=0)) == ssm.SSM_OK         # nothing to scan: no checkpoints


def bidir_bwd_ckpt(**kw):
    args = dict(BWD_DEFAULT)
    args.update(opts=None, Bs=2, L=64, ED=64, N=16, dtype=ssm.SSM_BF16, ck=P[24])
    args["ws_bytes"] = ssm.ssm_scan_bidir_bwd_workspace_bytes(2, 64, 64, 16, ssm.SSM_BF16)
    args["ck_bytes"] = ssm.lib().ssm_scan_ckpt_bytes(2, 64, 64, 16)
    args.update(kw)
    head = [args[n] for n in BIDIR_BWD_ORDER[:12]]
    tail = [args[n] for n in BIDIR_BWD_ORDER[12:]]
    return ssm.lib().ssm_scan_bidir_bwd_ckpt(*head, args["ck"], args["ck_bytes"], *tail, args["Bs"], args["L"],
                                             args["ED"], args["N"], args["dtype"], args["ws"], args["ws_bytes"], None)


def test_bidir_backward_checkpoint_validation():
    assert BIDIR_BWD_ORDER[11] == "dg_first" and BIDIR_BWD_ORDER[12] == "dx"
    assert bidir_bwd_ckpt(ck=None) == ssm.SSM_ERR_NULL
    assert bidir_bwd_ckpt(ck=P[24] + 4) == ssm.SSM_ERR_UNSUPPORTED       # misaligned
    assert bidir_bwd_ckpt(ck_bytes=64) == ssm.SSM_ERR_WORKSPACE          # too small
    assert bidir_bwd_ckpt(ck=P[9]) == ssm.SSM_ERR_ALIAS                  # dx on top of the checkpoints
    assert bidir_bwd_ckpt(ck=P[22]) == ssm.SSM_ERR_ALIAS                 # dg0 on top of them
    assert bidir_bwd_ckpt(ck=P[18]) == ssm.SSM_ERR_ALIAS                 # the workspace on top of them
    none = {n: None for n in BWD_PTRS}
    assert bidir_bwd_ckpt(**dict(none, ck=None, Bs=0, ED=0, ws_bytes=0)) == ssm.SSM_OK


def test_binding_checks_bidir_checkpoint_tensors():
    import torch
    x = torch.zeros(2, 40, 20)
    d, B, C = torch.zeros(2, 40, 20), torch.zeros(2, 40, 16), torch.zeros(2, 40, 16)
    A = torch.zeros(20, 16)
    with pytest.raises(ValueError, match="ckpt must have shape"):
        ssm.ssm_scan_bidir_fwd(x, d, A, B, C, ckpt=torch.zeros(2, 2, 20, 16))
    with pytest.raises(TypeError, match="ckpt must be torch.float32"):
        ssm.ssm_scan_bidir_fwd(x, d, A, B, C, ckpt=torch.zeros(2, 2, 32, 16, dtype=torch.float64))
    with pytest.raises(TypeError):
        ssm.ssm_scan_bidir_bwd(x, d, A, B, C, None, x, ckpt=torch.zeros(2, 2, 32, 16, dtype=torch.bfloat16))

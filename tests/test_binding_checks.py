"""The Python binding checks every tensor against x (dtype, shape, contiguity,
device) before it takes a pointer: the C ABI receives bare addresses and
sizes, so a float64 A, a transposed B or a short output would otherwise be
misread or overrun there. The checks run before the GPU check, so each
rejection shows on CPU tensors (no library call is made)."""
import pytest
import torch

import state_space_model_selective_amd as ssm

Bs, L, ED, N = 2, 8, 12, 16
f32, bf16 = torch.float32, torch.bfloat16


def scan_inputs(dtype=f32):
    g = torch.Generator().manual_seed(0)
    r = lambda *s, dt=dtype: torch.randn(*s, generator=g).to(dt)
    return dict(x=r(Bs, L, ED), delta=r(Bs, L, ED).abs(), A=-torch.rand(ED, N, generator=g) - 0.5,
                B=r(Bs, L, N), C=r(Bs, L, N), D=r(ED, dt=f32))


def gpu_only(fn, **kw):
    with pytest.raises(RuntimeError, match="GPU only"):
        fn(**kw)


# --- all arguments valid: only the GPU check remains ------------------------
@pytest.mark.parametrize("dtype", [f32, bf16])
def test_valid_cpu_arguments_reach_the_gpu_check(dtype):
    t = scan_inputs(dtype)
    gpu_only(ssm.ssm_scan_fwd, **t, h_last=torch.empty(Bs, ED, N), h0=torch.zeros(Bs, ED, N),
             dt_bias=torch.zeros(ED), z=torch.zeros(Bs, L, ED, dtype=dtype), dt_limit=(0.0, 1.0))
    gpu_only(ssm.ssm_scan_bidir_fwd, **t, g_first=torch.empty(Bs, ED, N))
    gpu_only(ssm.ssm_scan_bwd, **t, dy=torch.zeros(Bs, L, ED, dtype=dtype),
             out={"dx": torch.empty(Bs, L, ED, dtype=dtype), "dA": torch.empty(ED, N)})
    gpu_only(ssm.ssm_scan_bidir_bwd, **t, dy=torch.zeros(Bs, L, ED, dtype=dtype))


# --- one bad tensor at a time ------------------------------------------------
BAD_DTYPE = [("delta", lambda t: t["delta"].double()), ("B", lambda t: t["B"].to(bf16)),
             ("C", lambda t: t["C"].half()), ("A", lambda t: t["A"].double()), ("D", lambda t: t["D"].to(bf16))]


@pytest.mark.parametrize("name,bad", BAD_DTYPE)
def test_wrong_dtype(name, bad):
    t = scan_inputs()
    t[name] = bad(t)
    with pytest.raises((TypeError, ValueError), match=name):
        ssm.ssm_scan_fwd(**t)


@pytest.mark.parametrize("name,shape", [("delta", (Bs, L, ED + 1)), ("B", (Bs, L, N + 1)), ("C", (Bs, L + 1, N)),
                                        ("A", (ED + 1, N)), ("D", (ED - 1,))])
def test_wrong_shape(name, shape):
    t = scan_inputs()
    t[name] = torch.zeros(shape)
    with pytest.raises(ValueError, match=name):
        ssm.ssm_scan_fwd(**t)


@pytest.mark.parametrize("name", ["delta", "B", "C"])
def test_not_contiguous(name):
    t = scan_inputs()
    v = t[name]
    t[name] = v.transpose(1, 2).contiguous().transpose(1, 2)  # same shape, transposed layout
    assert not t[name].is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        ssm.ssm_scan_fwd(**t)


def test_transposed_A():
    t = scan_inputs()
    t["A"] = torch.zeros(N, ED).t()  # (ED, N) view of a transposed buffer
    with pytest.raises(ValueError, match="contiguous"):
        ssm.ssm_scan_fwd(**t)


@pytest.mark.parametrize("name", ["delta", "B", "D"])
def test_other_device(name):
    t = scan_inputs()
    t[name] = torch.empty(t[name].shape, dtype=t[name].dtype, device="meta")
    with pytest.raises(ValueError, match="device|meta"):
        ssm.ssm_scan_fwd(**t)


def test_x_itself():
    t = scan_inputs()
    with pytest.raises(TypeError):
        ssm.ssm_scan_fwd(**dict(t, x=t["x"].double()))
    with pytest.raises(ValueError):
        ssm.ssm_scan_fwd(**dict(t, x=t["x"][0]))
    with pytest.raises(TypeError):
        ssm.ssm_scan_fwd(**dict(t, x=t["x"].numpy()))


@pytest.mark.parametrize("kw", [
    dict(y=torch.empty(Bs, L, ED - 1)),
    dict(y=torch.empty(Bs, L, ED, dtype=bf16)),
    dict(h_last=torch.empty(Bs, ED, N + 1)),
    dict(h_last=torch.empty(Bs, ED, N, dtype=torch.float64)),
    dict(h0=torch.zeros(Bs, N, ED)),
    dict(dt_bias=torch.zeros(ED, 1)),
    dict(z=torch.zeros(Bs, L, ED, dtype=bf16)),
    dict(dt_limit=(0.0, 1.0, 2.0)),
    dict(workspace=torch.empty(64, dtype=torch.uint8, device="meta")),
])
def test_forward_outputs_and_options(kw):
    with pytest.raises((TypeError, ValueError)):
        ssm.ssm_scan_fwd(**scan_inputs(), **kw)


def test_bidirectional_g_first():
    with pytest.raises(ValueError, match="g_first"):
        ssm.ssm_scan_bidir_fwd(**scan_inputs(), g_first=torch.empty(Bs, ED, N - 1))


@pytest.mark.parametrize("out", [
    {"dx": torch.empty(Bs, L, ED, dtype=bf16)},
    {"ddelta": torch.empty(Bs, L + 1, ED)},
    {"dA": torch.empty(ED, N, dtype=torch.float64)},
    {"dB": torch.empty(Bs, L, N - 1)},
    {"dC": torch.empty(Bs, N, L).transpose(1, 2)},
    {"dD": torch.empty(ED + 1)},
    {"dh0": torch.empty(Bs, ED, N, dtype=bf16)},
    {"ddt_bias": torch.empty(ED, 2)},
    {"dz": torch.empty(Bs, L, ED, dtype=torch.float64)},
    {"dq": torch.empty(1)},
])
def test_backward_outputs(out):
    t = scan_inputs()
    with pytest.raises((TypeError, ValueError)):
        ssm.ssm_scan_bwd(**t, dy=torch.zeros(Bs, L, ED), out=out)


def test_backward_dy():
    t = scan_inputs()
    with pytest.raises(TypeError, match="dy"):
        ssm.ssm_scan_bwd(**t, dy=torch.zeros(Bs, L, ED, dtype=bf16))
    with pytest.raises(ValueError, match="dy"):
        ssm.ssm_scan_bidir_bwd(**t, dy=torch.zeros(Bs, L, ED + 1))
    with pytest.raises(ValueError, match="dy"):
        ssm.ssm_scan_bwd(**t, dy=None)


# --- multi-head scan ----------------------------------------------------------
H, P, G, NS = 4, 64, 2, 128


def ssd_inputs(dtype=f32):
    g = torch.Generator().manual_seed(1)
    r = lambda *s, dt=dtype: torch.randn(*s, generator=g).to(dt)
    return dict(x=r(Bs, L, H, P), dt=r(Bs, L, H).abs(), A=-torch.rand(H, generator=g), B=r(Bs, L, G, NS),
                C=r(Bs, L, G, NS), D=r(H, dt=f32))


def test_ssd_valid_cpu_arguments_reach_the_gpu_check():
    gpu_only(ssm.ssm_ssd_fwd, **ssd_inputs(), h_last=torch.empty(Bs, H, P, NS))
    gpu_only(ssm.ssm_ssd_bidir_fwd, **ssd_inputs(bf16), g_first=torch.empty(Bs, H, P, NS))


@pytest.mark.parametrize("name,value", [
    ("dt", torch.zeros(Bs, L, H + 1)), ("A", torch.zeros(H, dtype=torch.float64)), ("B", torch.zeros(Bs, L, G, NS, 1)),
    ("C", torch.zeros(Bs, L, G, NS + 1)), ("D", torch.zeros(H + 1)), ("x", torch.zeros(Bs, L, H)),
])
def test_ssd_rejections(name, value):
    t = ssd_inputs()
    t[name] = value
    with pytest.raises((TypeError, ValueError)):
        ssm.ssm_ssd_fwd(**t)


def test_ssd_outputs():
    t = ssd_inputs()
    with pytest.raises(ValueError, match="h_last"):
        ssm.ssm_ssd_fwd(**t, h_last=torch.empty(Bs, H, NS, P))
    with pytest.raises(TypeError, match="y"):
        ssm.ssm_ssd_bidir_fwd(**t, y=torch.empty(Bs, L, H, P, dtype=bf16))

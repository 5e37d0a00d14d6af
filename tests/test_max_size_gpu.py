"""Scans whose tensors hold more than 2^31 elements (x, delta and y over 8 GiB
each in float32), through the C ABI, against the fp64 oracle on sampled
channels (every time step of each).

Element offsets past 2^31 and byte offsets past 2^32 must be formed in 64
bits everywhere: in the staging loads, the output stores, the final-state
stores and the split sequence's hand-off. The shape also has a ragged last
channel group (ED = 2060 = 128 * 16 + 12), and with one batch row the
forward scan splits the sequence across workgroups. Inputs come from the
seeded generator with the workloads' distributions (x, B, C, D ~ N(0,1),
delta log-uniform on [1e-3, 1e-1], A[e, n] = -(n+1)).
"""
import numpy as np
import pytest

import oracle
import synth
from parity_util import TOL, assert_close, log

pytestmark = pytest.mark.gpu

Bs, L, ED, N = 1, 1_052_675, 2060, 16
# channels b * ED + e to check: the first and last of the first and last
# groups, one inside, and the last channel of the ragged group
CHANS = np.array([0, 7, 1023, 2047, 2048, 2059], dtype=np.int64)


@pytest.fixture(scope="module")
def big():
    import torch
    assert Bs * L * ED > 2 ** 31
    log("max-size inputs: Bs=%d L=%d ED=%d (%d elements per tensor)" % (Bs, L, ED, Bs * L * ED))
    inp = synth.make_inputs(Bs, L, ED, N, "f32", seed=5)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(v).to(dev) for k, v in inp.items()}
    log("max-size inputs on the device")
    yield inp, t
    del t
    torch.cuda.empty_cache()


def sampled(y):
    """(len(CHANS), L) float64 of the device output y (Bs, L, ED)."""
    import torch
    b, e = np.divmod(CHANS, ED)
    idx = torch.from_numpy(e).to(y.device)
    return y[int(b[0])].index_select(1, idx).t().double().cpu().numpy()


def test_forward_beyond_2_31_elements(big):
    import torch
    import state_space_model_selective_amd as ssm
    inp, t = big
    h = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device="cuda:0")
    y = ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], h_last=h)
    torch.cuda.synchronize()
    log("max-size forward done")
    assert bool(torch.isfinite(y).all())
    y_ref, h_ref, _ = oracle.scan(**inp, chans=CHANS, want_h_last=True)
    assert_close("y[sampled channels]", sampled(y), y_ref, TOL["f32"])
    b, e = np.divmod(CHANS, ED)
    assert_close("h_last[sampled]", h.double().cpu().numpy()[b, e], h_ref, TOL["f32"])
    del y, h


def test_bidirectional_beyond_2_31_elements(big):
    import torch
    import state_space_model_selective_amd as ssm
    inp, t = big
    g = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device="cuda:0")
    y = ssm.ssm_scan_bidir_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], g_first=g)
    torch.cuda.synchronize()
    log("max-size bidirectional done")
    assert bool(torch.isfinite(y).all())
    y_ref, _, g_ref = oracle.scan(**inp, bidir=True, chans=CHANS, want_g_first=True)
    assert_close("y[sampled channels]", sampled(y), y_ref, TOL["f32"])
    b, e = np.divmod(CHANS, ED)
    assert_close("g_first[sampled]", g.double().cpu().numpy()[b, e], g_ref, TOL["f32"])
    del y, g


def test_backward_beyond_2_31_elements():
    """Backward pass over 4 x 32771 x 16388 channels (2^31 + 720,944 elements
    per tensor). dy is zero except on a few sampled channels: every other
    channel's adjoint is then exactly zero, so its dx, ddelta, dA and dD are
    exact zeros and the full-size dB and dC (sums over all channels, whose
    per-group partials also pass 2^31 elements) equal the oracle's on the
    sampled channels alone."""
    import torch
    import state_space_model_selective_amd as ssm
    Bs_, L_, ED_ = 4, 32771, 16388
    assert Bs_ * L_ * ED_ > 2 ** 31
    es = np.array([0, 15, 8191, 16383, 16384, 16387], dtype=np.int64)  # 16388 = 1024 * 16 + 4: a ragged group
    log("max-size backward: Bs=%d L=%d ED=%d" % (Bs_, L_, ED_))
    inp = synth.make_inputs(Bs_, L_, ED_, N, "f32", seed=6)
    dy_s = synth.normal(6, 41, (Bs_, L_, es.size))
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(v).to(dev) for k, v in inp.items()}
    eidx = torch.from_numpy(es).to(dev)
    dy = torch.zeros((Bs_, L_, ED_), dtype=torch.float32, device=dev)
    dy.index_copy_(2, eidx, torch.from_numpy(dy_s).to(dev))
    res = ssm.ssm_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], dy)
    torch.cuda.synchronize()
    log("max-size backward done")
    sub = {k: (np.ascontiguousarray(v[:, :, es]) if k in ("x", "delta") else v) for k, v in inp.items()}
    sub["A"] = np.ascontiguousarray(inp["A"][es])
    sub["D"] = np.ascontiguousarray(inp["D"][es])
    ref = oracle.scan_bwd(**sub, dy=dy_s)
    for k in ("dx", "ddelta"):
        got = res[k].index_select(2, eidx).double().cpu().numpy()
        assert_close(k + "[sampled channels]", got, ref[k], TOL["f32"])
        res[k].index_fill_(2, eidx, 0.0)
        assert int(torch.count_nonzero(res[k])) == 0, "%s is not zero on channels without output gradient" % k
    for k in ("dA", "dD"):
        got = res[k].index_select(0, eidx).double().cpu().numpy()
        assert_close(k + "[sampled channels]", got, ref[k], TOL["f32"])
        res[k].index_fill_(0, eidx, 0.0)
        assert int(torch.count_nonzero(res[k])) == 0, "%s is not zero on channels without output gradient" % k
    for k in ("dB", "dC"):
        assert_close(k, res[k].double().cpu().numpy(), ref[k], TOL["f32"])
    del t, dy, res
    torch.cuda.empty_cache()


def test_multihead_beyond_2_31_elements():
    """bf16 multi-head scan with x of 8 x 65601 x 64 heads x 64 (2^31 + 1,474,560
    elements, 4.3 GB), one B/C group (every head independent), against the
    oracle on sampled (batch row, head) pairs, the last one included."""
    import torch
    import state_space_model_selective_amd as ssm
    Bs_, L_, H, P, G, Nh = 8, 65601, 64, 64, 1, 128
    assert Bs_ * L_ * H * P > 2 ** 31
    log("max-size multi-head: Bs=%d L=%d H=%d P=%d N=%d bf16" % (Bs_, L_, H, P, Nh))
    inp = synth.make_ssd_inputs(Bs_, L_, H, P, G, Nh, "bf16", seed=7)
    dev = torch.device("cuda:0")

    def dev_t(v):
        if v.dtype == np.uint16:
            return torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(v).to(dev)

    t = {k: dev_t(v) for k, v in inp.items()}
    hl = torch.full((Bs_, H, P, Nh), float("nan"), dtype=torch.float32, device=dev)
    y = ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], h_last=hl)
    torch.cuda.synchronize()
    log("max-size multi-head done")
    for b, h in ((0, 0), (3, 41), (7, 63)):
        sub = dict(x=np.ascontiguousarray(inp["x"][b:b + 1, :, h:h + 1]),
                   dt=np.ascontiguousarray(inp["dt"][b:b + 1, :, h:h + 1]),
                   A=inp["A"][h:h + 1].copy(), B=np.ascontiguousarray(inp["B"][b:b + 1]),
                   C=np.ascontiguousarray(inp["C"][b:b + 1]), D=inp["D"][h:h + 1].copy())
        y_ref, h_ref, _ = oracle.ssd(**sub, want_h_last=True)
        got = y[b:b + 1, :, h:h + 1].float().cpu().numpy().astype(np.float64)
        assert_close("y[b=%d, head %d]" % (b, h), got, y_ref, TOL["bf16"])
        assert_close("h_last[b=%d, head %d]" % (b, h), hl[b:b + 1, h:h + 1].double().cpu().numpy(), h_ref,
                     TOL["f32"])
    del t, y, hl
    torch.cuda.empty_cache()

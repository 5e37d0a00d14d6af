"""ssm_scan_fwd_noalloc, the forward scan for callers that cannot allocate:
called through the C ABI, it must give the same output as ssm_scan_fwd (the
same kernels run, so bit for bit, and within the oracle's tolerance), on two
calls in a row, the second with a smaller input (the library's device buffer
keeps the first call's contents, which must not leak into the second)."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import TOL, assert_close, log, to_device, y_to_numpy

pytestmark = pytest.mark.gpu


def run_both(Bs, L, ED, dtype, seed):
    import torch
    import state_space_model_selective_amd as ssm
    N = 16
    log("case no-alloc %dx%dx%d %s seed %d" % (Bs, L, ED, dtype, seed))
    inp = synth.make_inputs(Bs, L, ED, N, dtype, seed=seed)
    dev = torch.device("cuda:0")
    t = to_device(inp, dev)
    code = ssm.SSM_F32 if dtype == "f32" else ssm.SSM_BF16
    need = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, code)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    y_ref_gpu = torch.empty_like(t["x"])
    h_ref_gpu = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev)
    ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=y_ref_gpu, h_last=h_ref_gpu,
                     workspace=ws)
    # the entry point under test, called through the C ABI with caller-owned outputs
    y = torch.full_like(t["x"], float("nan"))
    h = torch.full((Bs, ED, N), float("nan"), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = ssm.lib().ssm_scan_fwd_noalloc(t["x"].data_ptr(), t["delta"].data_ptr(), t["A"].data_ptr(),
                                        t["B"].data_ptr(), t["C"].data_ptr(), t["D"].data_ptr(), None, None,
                                        y.data_ptr(), h.data_ptr(), Bs, L, ED, N, code, stream)
    assert rc == ssm.SSM_OK, ssm.status_str(rc)
    assert ssm.ssm_scan_fwd_status(t["x"], t["A"], None) == ssm.SSM_OK
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref_gpu), "no-alloc output differs from ssm_scan_fwd"
    assert torch.equal(h, h_ref_gpu), "no-alloc final state differs from ssm_scan_fwd"
    y_ref, h_ref, _ = oracle.scan(**inp, want_h_last=True)
    assert_close("y", y_to_numpy(y), y_ref, TOL[dtype])
    assert_close("h_last", h.double().cpu().numpy(), h_ref, TOL["f32"])
    return need


def test_two_calls_second_smaller():
    # a split sequence (the library's buffer is used), then a smaller split one
    n1 = run_both(1, 20000, 128, "f32", seed=31)
    n2 = run_both(1, 9000, 64, "f32", seed=32)
    assert n1 > 0 and n2 > 0 and n2 < n1


def test_unsplit_and_bf16():
    # shapes that need no hand-off buffer, and a bf16 split sequence
    run_both(2, 300, 64, "f32", seed=33)
    run_both(2, 4096, 32, "bf16", seed=34)
    run_both(1, 20000, 128, "f32", seed=35)


def test_wrapper_and_errors():
    import torch
    import state_space_model_selective_amd as ssm
    inp = synth.make_inputs(1, 3000, 64, 16, "f32", seed=36)
    t = to_device(inp, torch.device("cuda:0"))
    y = ssm.ssm_scan_fwd_noalloc(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"])
    y_ref, _, _ = oracle.scan(**inp)
    assert_close("y", y_to_numpy(y), y_ref, TOL["f32"])
    # argument errors are reported like ssm_scan_fwd's, before any launch
    rc = ssm.lib().ssm_scan_fwd_noalloc(None, t["delta"].data_ptr(), t["A"].data_ptr(), t["B"].data_ptr(),
                                        t["C"].data_ptr(), None, None, None, y.data_ptr(), None, 1, 3000, 64, 16,
                                        ssm.SSM_F32, None)
    assert rc == ssm.SSM_ERR_NULL
    rc = ssm.lib().ssm_scan_fwd_noalloc(t["x"].data_ptr(), t["delta"].data_ptr(), t["A"].data_ptr(),
                                        t["B"].data_ptr(), t["C"].data_ptr(), None, None, None, y.data_ptr(), None,
                                        1, 3000, 64, 8, ssm.SSM_F32, None)
    assert rc == ssm.SSM_ERR_UNSUPPORTED
    assert ssm.SSM_NOALLOC_SCRATCH_BYTES == 1 << 20
    assert ssm.ssm_scan_workspace_bytes(1, 1 << 20, 16, 16) <= ssm.SSM_NOALLOC_SCRATCH_BYTES

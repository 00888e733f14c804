"""Hand-offs between waves and workgroups under stress, through the C ABI.

Bounded waits: with the wait limit forced down to one poll from the host
(sdtw_debug_wait_limit), the waits of every mode give up; every kernel still
exits normally, the outputs of the call are NaN and the workspace reports
SDTW_ERR_STALLED.  With the limit restored the same workspace gives bitwise
the results of an untouched one."""
import numpy as np
import pytest
import torch

from sdtw_inputs import pair_batch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def L():
    from differentiable_series_alignment_amd import _lib
    _lib.lib()   # loud failure if the HIP library is missing
    return _lib


def run(L, mode, x, y, gamma, ws, grads=True):
    B, N, D = x.shape
    M = y.shape[1]
    s = torch.cuda.current_stream().cuda_stream
    loss = torch.empty(B, device=DEV)
    L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                           ws.data_ptr(), ws.numel(), loss.data_ptr(), s), "sdtw_forward")
    gx = gy = None
    if grads and mode != L.SDTW_MODE_INFERENCE:
        gx, gy = torch.empty_like(x), torch.empty_like(y)
        gl = torch.full((B,), 1.0 / B, device=DEV)
        L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                                ws.data_ptr(), ws.numel(), gl.data_ptr(), gx.data_ptr(),
                                gy.data_ptr(), None, s), "sdtw_backward")
    st = L.sdtw_workspace_status(ws.data_ptr(), ws.numel(), B, N, M, D, mode, s)
    return st, loss, gx, gy


@pytest.mark.parametrize("mode,shape", [
    (0, (4, 300, 500, 8)),     # unfused: 4-band workgroups, two segments
    (1, (3, 200, 300, 8)),     # fused: one band per workgroup
    (2, (3, 1100, 700, 5)),    # inference through 512-column rings
    (2, (3, 130, 90, 4)),      # inference with whole rows
    (3, (2, 300, 200, 5)),     # checkpointed training
    (4, (4, 300, 500, 8)),     # low-memory unfused: forward sweep, then the E-forming reverse
])
def test_wait_giveup_is_reported(L, mode, shape):
    B, N, M, D = shape
    x, y = (t.to(DEV) for t in pair_batch(B, N, M, D, seed=N + M))
    nb = L.sdtw_workspace_bytes(B, N, M, D, mode)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    print(f"mode {mode} shape {shape}: wait limit 1", flush=True)
    try:
        assert L.sdtw_debug_wait_limit(1) == L.SDTW_OK
        st, loss, gx, gy = run(L, mode, x, y, 0.5, ws)
        torch.cuda.synchronize()
    finally:
        L.sdtw_debug_wait_limit(0)
    assert st == L.SDTW_ERR_STALLED
    assert torch.isnan(loss).all()
    if gx is not None:
        assert torch.isnan(gx).all() and torch.isnan(gy).all()
    # Normal limits again: the same workspace and a fresh one agree bitwise.
    st2, loss2, gx2, gy2 = run(L, mode, x, y, 0.5, ws)
    ws_fresh = torch.empty(nb, dtype=torch.uint8, device=DEV)
    st3, loss3, gx3, gy3 = run(L, mode, x, y, 0.5, ws_fresh)
    torch.cuda.synchronize()
    assert st2 == L.SDTW_OK and st3 == L.SDTW_OK
    assert torch.isfinite(loss2).all()
    torch.testing.assert_close(loss2, loss3, rtol=0, atol=0)
    if gx2 is not None:
        torch.testing.assert_close(gx2, gx3, rtol=0, atol=0)
        torch.testing.assert_close(gy2, gy3, rtol=1e-5, atol=1e-7)

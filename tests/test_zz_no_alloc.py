"""The allocation-free loss-only entry point (sdtw_forward_static) through
the C ABI: bitwise the loss of sdtw_forward in inference mode with a caller
workspace, on two calls in a row (the second on a smaller problem, so it
finds the first call's contents in the shared device array), rejection of a
problem whose workspace exceeds the array, and no device allocation."""
import pytest
import torch

from sdtw_inputs import pair_batch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _lib():
    from differentiable_series_alignment_amd import _lib as L
    L.lib()   # loud failure if the HIP library is missing
    return L


def _reference_loss(L, x, y, gamma, s):
    B, N, D = x.shape
    M = y.shape[1]
    nb = L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_INFERENCE)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    loss = torch.empty(B, device=DEV)
    L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma,
                           L.SDTW_MODE_INFERENCE, ws.data_ptr(), nb, loss.data_ptr(), s),
            "sdtw_forward")
    return loss


def test_static_forward_matches_inference_mode():
    L = _lib()
    s = torch.cuda.current_stream().cuda_stream
    # (8, 700, 600, 16): 512-column rings; (3, 100, 90, 4): whole rows.
    shapes = [(8, 700, 600, 16, 0.7), (3, 100, 90, 4, 1.3)]
    inputs = [tuple(t.to(DEV) for t in pair_batch(B, N, M, D, seed=N + M)) + (g,)
              for (B, N, M, D, g) in shapes]
    refs = [_reference_loss(L, x, y, g, s) for (x, y, g) in inputs]
    outs = [torch.full((x.shape[0],), float("nan"), device=DEV) for (x, _, _) in inputs]
    torch.cuda.synchronize()
    for k, (x, y, g) in enumerate(inputs):
        B, N, D = x.shape
        M = y.shape[1]
        assert L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_INFERENCE) <= \
            L.SDTW_STATIC_SCRATCH_BYTES
        free0 = torch.cuda.mem_get_info()[0]
        L.check(L.sdtw_forward_static(x.data_ptr(), y.data_ptr(), B, N, M, D, g,
                                      outs[k].data_ptr(), s), "sdtw_forward_static")
        torch.cuda.synchronize()
        if k > 0:   # the first call may load the code object; later ones allocate nothing
            assert torch.cuda.mem_get_info()[0] == free0
        torch.testing.assert_close(outs[k], refs[k], rtol=0, atol=0)
    # the same problem again after the smaller one: still bitwise the same
    x, y, g = inputs[0]
    again = torch.empty(x.shape[0], device=DEV)
    L.check(L.sdtw_forward_static(x.data_ptr(), y.data_ptr(), x.shape[0], x.shape[1],
                                  y.shape[1], x.shape[2], g, again.data_ptr(), s),
            "sdtw_forward_static")
    torch.cuda.synchronize()
    torch.testing.assert_close(again, refs[0], rtol=0, atol=0)


def test_static_forward_rejects_beyond_limit():
    L = _lib()
    # 64 pairs of 8192 x 500: whole hand-off rows, 64*128*500*8 B = 31 MiB.
    B, N, M, D = 64, 8192, 500, 2
    need = L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_INFERENCE)
    assert need > L.SDTW_STATIC_SCRATCH_BYTES
    x = torch.zeros(1, device=DEV)
    st = L.sdtw_forward_static(x.data_ptr(), x.data_ptr(), B, N, M, D, 1.0, x.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == L.SDTW_ERR_WORKSPACE
    assert L.sdtw_forward_static(None, x.data_ptr(), 1, 1, 1, 1, 1.0, x.data_ptr(), 0) == \
        L.SDTW_ERR_INVALID_ARG

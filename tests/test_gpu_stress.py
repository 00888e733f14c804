"""Hand-off protocols under pseudo-random delays, through the C ABI.

libsdtw_stress.so is the library built from the same sources with
SDTW_STRESS=1: every producer's publish, every consumer's wait and every
pass of a hand-off wave (LDS rings between band waves, global rows and rings
between workgroups, the fused band waves' direct row stores) first sleeps a
pseudo-random time of up to ~13 us.  Producers and consumers then meet in
orders the normal build rarely shows.  The results may not change: losses,
dx and (where it is summed in a fixed order) dy are bitwise those of the
normal build, the rest to rounding, and no wait gives up.  Each case runs
twice on the stress build; the run stops at the first mismatch."""
import pytest
import torch

from sdtw_inputs import pair_batch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def libs():
    from differentiable_series_alignment_amd import _lib
    return _lib, _lib.lib(), _lib.load(_lib.STRESS_LIB_PATH)


def step(L, h, mode, x, y, gamma):
    """One forward (+ backward unless inference) on build `h`; returns the
    workspace status, the loss and the gradients."""
    B, N, D = x.shape
    M = y.shape[1]
    nb = h.sdtw_workspace_bytes(B, N, M, D, mode)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    loss = torch.empty(B, device=DEV)
    assert h.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode, ws.data_ptr(),
                          nb, loss.data_ptr(), s) == L.SDTW_OK
    gx = gy = None
    if mode != L.SDTW_MODE_INFERENCE:
        gx, gy = torch.empty_like(x), torch.empty_like(y)
        gl = torch.full((B,), 1.0 / B, device=DEV)
        assert h.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                               ws.data_ptr(), nb, gl.data_ptr(), gx.data_ptr(), gy.data_ptr(),
                               None, s) == L.SDTW_OK
    st = h.sdtw_workspace_status(ws.data_ptr(), nb, B, N, M, D, mode, s)
    torch.cuda.synchronize()
    return st, loss, gx, gy


CASES = [
    (0, (3, 70, 45, 3)),        # unfused: one ragged band
    (0, (2, 300, 700, 5)),      # unfused: bands of one workgroup, ragged edges
    (0, (3, 1100, 700, 5)),     # unfused: several segments per pair
    (0, (32, 512, 512, 64)),    # unfused: the headline batch
    (1, (3, 70, 45, 3)),        # fused
    (1, (2, 300, 700, 5)),
    (1, (32, 512, 512, 64)),
    (2, (3, 70, 45, 3)),        # inference, whole rows
    (2, (3, 1100, 700, 5)),     # inference through 512-column rings
    (3, (3, 1100, 700, 5)),     # checkpointed training (group launches)
    (3, (2, 2100, 300, 4)),
    (4, (3, 1100, 700, 5)),     # low-memory unfused: forward, then the E-forming reverse
    (4, (32, 512, 512, 64)),
]


@pytest.mark.parametrize("mode,shape", CASES)
def test_stress_build_matches_normal_build(libs, mode, shape):
    L, h0, h1 = libs
    B, N, M, D = shape
    x, y = (t.to(DEV) for t in pair_batch(B, N, M, D, seed=N + 3 * M + D))
    gamma = 0.7
    print(f"stress: mode {mode} shape {shape}", flush=True)
    st0, l0, gx0, gy0 = step(L, h0, mode, x, y, gamma)
    assert st0 == L.SDTW_OK
    for rep in range(2):
        print(f"  stress build, run {rep}", flush=True)
        st, l1, gx1, gy1 = step(L, h1, mode, x, y, gamma)
        assert st == L.SDTW_OK, L.sdtw_status_string(st)
        torch.testing.assert_close(l1, l0, rtol=0, atol=0)
        if gx0 is not None:
            torch.testing.assert_close(gx1, gx0, rtol=0, atol=0)
            if mode in (L.SDTW_MODE_UNFUSED, L.SDTW_MODE_UNFUSED_LOWMEM):
                torch.testing.assert_close(gy1, gy0, rtol=0, atol=0)
            else:   # dy through fp32 atomics: order of the sums varies
                torch.testing.assert_close(gy1, gy0, rtol=1e-5, atol=1e-6)

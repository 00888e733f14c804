"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sdtw.h, and rejects invalid calls on the host before any
HIP call (README "SoftDTW-CUDA (PyTorch + Numba)", "Tests": validation of
gamma, device, empty sequences and shape mismatches)."""
import ctypes
import os
import re

import pytest
import torch

from differentiable_series_alignment_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdtw.h")
FAKE = 1 << 20  # a non-null address that must never be dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sdtw_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(L.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert L.sdtw_abi_version() == 3


def test_stress_build_exports_the_same_symbols():
    """The hand-off stress build (same sources, SDTW_STRESS=1) loads and
    exports every declared entry point, with the same workspace sizes."""
    h = L.load(L.STRESS_LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name
    assert h.sdtw_abi_version() == L.sdtw_abi_version()
    for mode in range(4):
        assert (h.sdtw_workspace_bytes(32, 512, 512, 64, mode)
                == L.sdtw_workspace_bytes(32, 512, 512, 64, mode))


def test_status_strings():
    for st in range(0, 6):
        s = L.sdtw_status_string(st)
        assert isinstance(s, str) and s
    assert L.sdtw_status_string(L.SDTW_OK) == "ok"


def test_workspace_bytes():
    a = L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_UNFUSED)
    b = L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_FUSED)
    cells = 32 * 512 * 512
    assert a % 256 == 0 and b % 256 == 0
    assert a >= cells * 12 and b >= cells * 8 and b < a
    for bad in [(0, 4, 4, 1), (1, 0, 4, 1), (1, 4, 0, 1), (1, 4, 4, 0), (-1, 4, 4, 1)]:
        assert L.sdtw_workspace_bytes(*bad, L.SDTW_MODE_UNFUSED) == 0
    assert L.sdtw_workspace_bytes(1, 4, 4, 1, 7) == 0
    # fused mode keeps a band's x rows on chip: D up to 256
    assert L.sdtw_workspace_bytes(2, 100, 100, 256, L.SDTW_MODE_FUSED) > 0
    assert L.sdtw_workspace_bytes(2, 100, 100, 257, L.SDTW_MODE_FUSED) == 0


def _fwd(**kw):
    a = dict(x=FAKE, y=FAKE, B=2, N=4, M=5, D=3, gamma=1.0, mode=0,
             workspace=FAKE * 256, workspace_bytes=1 << 30, loss=FAKE, stream=0)
    a.update(kw)
    return L.sdtw_forward(**a)


def _bwd(**kw):
    a = dict(x=FAKE, y=FAKE, B=2, N=4, M=5, D=3, gamma=1.0, mode=0,
             workspace=FAKE * 256, workspace_bytes=1 << 30, grad_loss=FAKE,
             grad_x=FAKE, grad_y=FAKE, align=None, stream=0)
    a.update(kw)
    return L.sdtw_backward(**a)


@pytest.mark.parametrize("kw", [
    dict(gamma=0.0), dict(gamma=-1.0), dict(gamma=float("nan")), dict(gamma=float("inf")),
    dict(B=0), dict(N=0), dict(M=0), dict(D=0), dict(N=-3),
    dict(x=None), dict(y=None), dict(mode=5), dict(mode=-1), dict(workspace=None),
    dict(workspace=FAKE * 256 + 8),
])
def test_forward_backward_reject_invalid(kw):
    if "loss" not in kw:
        assert _fwd(**kw) == L.SDTW_ERR_INVALID_ARG
    assert _bwd(**kw) == L.SDTW_ERR_INVALID_ARG


def test_null_outputs_rejected():
    assert _fwd(loss=None) == L.SDTW_ERR_INVALID_ARG
    assert _bwd(grad_loss=None) == L.SDTW_ERR_INVALID_ARG


def test_small_workspace_rejected():
    need = L.sdtw_workspace_bytes(2, 4, 5, 3, 0)
    assert _fwd(workspace_bytes=need - 1) == L.SDTW_ERR_WORKSPACE
    assert _bwd(workspace_bytes=need - 256) == L.SDTW_ERR_WORKSPACE


def test_dist_rejects_invalid():
    assert L.sdtw_dist(None, FAKE, FAKE, 1, 2, 2, 2) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_dist(FAKE, FAKE, None, 1, 2, 2, 2) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_dist(FAKE, FAKE, FAKE, 1, 0, 2, 2) == L.SDTW_ERR_INVALID_ARG


# --- Python layer ---------------------------------------------------------------

def test_python_layer_validation_on_cpu():
    from differentiable_series_alignment_amd import SoftDTW, soft_dtw
    x = torch.randn(2, 5, 3)
    y = torch.randn(2, 6, 3)
    with pytest.raises(ValueError, match="GPU"):
        soft_dtw(x, y)                                  # no CPU path
    with pytest.raises(ValueError, match="sqeuclidean"):
        SoftDTW(dist="euclidean")
    with pytest.raises(ValueError, match="gamma"):
        SoftDTW(gamma=0.0)
    with pytest.raises(ValueError, match="gamma"):
        soft_dtw(x, y, gamma=-1.0)
    with pytest.raises(ValueError, match="batch"):
        soft_dtw(x, torch.randn(3, 6, 3))
    with pytest.raises(ValueError, match="feature"):
        soft_dtw(x, torch.randn(2, 6, 4))
    with pytest.raises(ValueError, match="empty"):
        soft_dtw(x, torch.randn(2, 0, 3))
    with pytest.raises(ValueError, match="float32"):
        soft_dtw(x.double(), y.double())
    with pytest.raises(ValueError, match="shape"):
        SoftDTW(normalize=True)(x, y)
    with pytest.raises(ValueError):
        soft_dtw(x[0], y[0])                            # not 3-D


def test_fused_choice_and_early_stopping_validation():
    from differentiable_series_alignment_amd import EarlyStopping, SoftDTW, choose_fused
    assert choose_fused(True, 2, 4, 4, 1) is True
    assert choose_fused(False, 2, 4, 4, 1) is False
    with pytest.raises(ValueError, match="fused"):
        choose_fused("yes", 2, 4, 4, 1)
    with pytest.raises(ValueError, match="fused"):
        SoftDTW(fused="maybe")
    with pytest.raises(ValueError):
        EarlyStopping(patience=0)
    es = EarlyStopping(patience=2, tol=0.0)
    assert [es.step(v) for v in (3.0, 2.0, 2.0, 2.5)] == [False, False, False, True]


def test_checkpoint_mode_workspace():
    """Checkpointed training keeps checkpoint rows and one group of bands'
    forward state (about sqrt(N/64) bands) instead of all N rows."""
    def ws(*a):
        return L.sdtw_workspace_bytes(*a, L.SDTW_MODE_CHECKPOINT)
    fused = L.sdtw_workspace_bytes(32, 4096, 4096, 128, L.SDTW_MODE_FUSED)
    assert 0 < ws(32, 4096, 4096, 128) * 5 < fused
    # the group of bands kept grows like sqrt(N): 4x the rows, about 2x the state
    r = ws(8, 16384, 1000, 4) / ws(8, 4096, 1000, 4)
    assert 1.7 < r < 2.5, r
    assert ws(2, 10, 10, 257) == 0 and ws(2, 10, 10, 256) > 0


def test_timing_switch_without_launches():
    """Launch timing can be switched and collected with nothing recorded (no
    HIP call is made then)."""
    assert L.sdtw_timing(True) == L.SDTW_OK
    assert L.sdtw_timing_collect() == []
    assert L.sdtw_timing(False) == L.SDTW_OK
    assert L.lib().sdtw_timing_collect(None, None, 0) == 0


def test_inference_mode_workspace_and_backward():
    """Inference mode: no B x N x M arrays, only the rows handed between
    64-row bands (whole, or 512-column rings once whole rows would be large
    or when every band fits on the GPU at once), D <= 256, and no backward."""
    def ws(*a):
        return L.sdtw_workspace_bytes(*a, L.SDTW_MODE_INFERENCE)
    train = L.sdtw_workspace_bytes(32, 4096, 4096, 128, L.SDTW_MODE_UNFUSED)
    infer = ws(32, 4096, 4096, 128)
    assert 0 < infer and infer * 100 < train
    rows = 32 * 64 * 4096 * 8                     # whole rows: 64 MiB < the inputs
    assert rows <= infer < rows + (1 << 20)
    # rings (every band fits at once): O(B*N), independent of M
    assert ws(4, 1000, 5000, 3) == ws(4, 1000, 9000, 3) < 4 * 16 * 512 * 8 + (1 << 16)
    # rings (whole rows would be 18.9 MB, above 16 MiB and the inputs)
    assert ws(9, 2048, 8192, 2) == ws(9, 2048, 9000, 2) < 9 * 32 * 512 * 8 + (1 << 16)
    # whole rows (small, and more bands than CUs)
    assert ws(40, 500, 600, 3) >= 40 * 8 * 600 * 8
    assert ws(2, 10, 10, 257) == 0
    assert _bwd(mode=L.SDTW_MODE_INFERENCE, D=3) == L.SDTW_ERR_UNSUPPORTED


def test_bench_step_bounds():
    """The per-configuration bounds bench.py reports, recomputed by hand for
    the headline workload (B=32, N=M=512, D=64): unfused distances 13.7 us
    (fp64 matrix), sweeps 42.6 us (1023 steps x 100 clocks at 2.4 GHz),
    chain rule 23.1 us (HBM, 20 B per cell plus twice the inputs); fused two
    sweeps of 42.6 us each.  And the JSON helpers add the fractions."""
    import bench
    B, N, M, D = 32, 512, 512, 64
    cells = B * N * M
    t_dist = 2 * cells * D / 78.6e12
    t_dp = (N + M - 1) * 100 / 2.4e9
    t_rule = (20 * cells + 2 * 4 * B * (N + M) * D) / 8e12
    u = bench.step_bounds(B, N, M, D, fused=False)
    assert abs(u["per_stage_us"] - 1e6 * (t_dist + t_dp + t_rule)) < 1e-6
    hbm = ((4 * cells + 4 * B * (N + M) * D) + 24 * cells
           + (20 * cells + 2 * 4 * B * (N + M) * D)) / 8e12
    assert abs(u["ideal_us"] - 1e6 * max(hbm, t_dp)) < 1e-6
    f = bench.step_bounds(B, N, M, D, fused=True)
    assert abs(f["per_stage_us"] - 2e6 * t_dp) < 1e-6
    e = bench.with_bounds({"ms_per_step": 0.2}, B, N, M, D, False)
    assert abs(e["frac_per_stage"] - u["per_stage_us"] / 200.0) < 1e-12
    assert abs(e["frac_ideal"] - u["ideal_us"] / 200.0) < 1e-12


def test_profile_summaries_name_their_commands():
    """Every rocprofv3 summary under profiles/ states the command that made
    it, and that command runs committed files only (bench.py with one of its
    own options)."""
    import sys
    import bench
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prof = os.path.join(root, "profiles")
    names = sorted(f for f in os.listdir(prof) if f.endswith(".md"))
    assert names
    for name in names:
        text = open(os.path.join(prof, name)).read()
        cmds = re.findall(r"rocprofv3 [^\n]*-- python3 bench\.py([^\n]*)", text)
        assert cmds, name
        for tail in cmds:
            argv = sys.argv
            try:
                sys.argv = ["bench.py"] + tail.split()
                bench.parse()
            except SystemExit as e:   # argparse rejects an unknown option
                raise AssertionError(f"{name}: bench.py {tail}") from e
            finally:
                sys.argv = argv


def test_status_query_and_wait_limit_validation():
    """The error-word query and the wait-limit hook reject bad arguments on
    the host; a valid query on a machine without a GPU fails in HIP, not
    silently."""
    B, N, M, D = 2, 100, 90, 3
    nb = L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_UNFUSED)
    assert L.sdtw_workspace_status(FAKE, nb, 0, N, M, D, L.SDTW_MODE_UNFUSED, 0) == \
        L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_workspace_status(FAKE, nb, B, N, M, D, 9, 0) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_workspace_status(FAKE, nb - 256, B, N, M, D, L.SDTW_MODE_UNFUSED, 0) == \
        L.SDTW_ERR_WORKSPACE
    assert L.sdtw_workspace_status(None, nb, B, N, M, D, L.SDTW_MODE_UNFUSED, 0) == \
        L.SDTW_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert L.sdtw_workspace_status(FAKE, nb, B, N, M, D, L.SDTW_MODE_UNFUSED, 0) == \
            L.SDTW_ERR_HIP
    assert L.sdtw_debug_wait_limit(-1) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_debug_wait_limit(1 << 32) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_debug_wait_limit(0) == L.SDTW_OK
    assert "gave up" in L.sdtw_status_string(L.SDTW_ERR_STALLED)


def test_low_memory_unfused_workspace():
    """The low-memory unfused mode keeps no reverse state: at least 8 bytes
    per cell less than the unfused mode and more than the fused one."""
    cells = 32 * 512 * 512
    unf = L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_UNFUSED)
    low = L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_UNFUSED_LOWMEM)
    fus = L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_FUSED)
    assert (unf - low) >= 8 * cells and low > fus > 0
    assert L.sdtw_workspace_bytes(2, 10, 10, 1000, L.SDTW_MODE_UNFUSED_LOWMEM) > 0   # any D
    assert L.sdtw_workspace_bytes(1, 4, 4, 1, 5) == 0


def test_unfused_band_stride():
    """The unfused arrays' bands are sweep_steps(M) = M + 63 rounded up to 16
    steps apart for any N (the steps a sweep runs outside the grid's columns
    reach no other band's cell), and the last band spans skew_steps(M) =
    M + 206 rounded: the reverse-state array, the one region the low-memory
    mode leaves out, holds ((bands - 1) * stride + skew) * 64 doubles."""
    def ws(B, N, M, mode):
        return L.sdtw_workspace_bytes(B, N, M, 8, mode)
    for B, N, M in [(4, 128, 1), (4, 127, 16), (3, 65, 17), (2, 1000, 100), (4, 64, 513),
                    (1, 1, 1), (2, 333, 1024)]:
        G = B * ((N + 63) // 64)
        stride = ((M + 78) // 16) * 16
        skew = ((M + 221) // 16) * 16
        t_bytes = ((G - 1) * stride + skew) * 64 * 8
        diff = ws(B, N, M, L.SDTW_MODE_UNFUSED) - ws(B, N, M, L.SDTW_MODE_UNFUSED_LOWMEM)
        assert diff == (t_bytes + 255) // 256 * 256, (B, N, M, diff, t_bytes)
    # ragged N costs nothing beyond its bands
    assert ws(4, 127, 100, 0) == ws(4, 128, 100, 0) == ws(4, 65, 100, 0)
    # the headline workload: B=32, N=M=512, D=64 (576-step bands)
    head = L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_UNFUSED)
    assert head < 190 << 20, head / 2**20
    assert L.sdtw_workspace_bytes(32, 512, 512, 64, L.SDTW_MODE_UNFUSED_LOWMEM) < 118 << 20


def test_static_forward_validation_on_host():
    """sdtw_forward_static rejects null pointers, bad sizes and problems whose
    inference workspace exceeds its device array before any HIP call."""
    assert L.sdtw_forward_static(None, FAKE, 1, 1, 1, 1, 1.0, FAKE, 0) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_forward_static(FAKE, FAKE, 0, 1, 1, 1, 1.0, FAKE, 0) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_forward_static(FAKE, FAKE, 2, 8, 8, 300, 1.0, FAKE, 0) == L.SDTW_ERR_INVALID_ARG
    assert L.sdtw_workspace_bytes(64, 8192, 500, 2, L.SDTW_MODE_INFERENCE) > \
        L.SDTW_STATIC_SCRATCH_BYTES
    assert L.sdtw_forward_static(FAKE, FAKE, 64, 8192, 500, 2, 1.0, FAKE, 0) == \
        L.SDTW_ERR_WORKSPACE

"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (fp32 results vs fp64 oracle): loss |l - l0| <= 1e-4 |l0| + 1e-5;
gradients |g - g0| <= 1e-5 + 1e-3 |g0| elementwise; no NaN/inf anywhere,
including gamma = 0.01.  The oracle reads Dist as the fp32 tensor it is in
the unfused mode: the exact squared distance rounded once to fp32.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from _pins import log_delannoy, zero_dist_marginals
from sdtw_inputs import block_waves, pair_batch

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DEV = "cuda:0"


@pytest.fixture(scope="module")
def S():
    import differentiable_series_alignment_amd as pkg
    from differentiable_series_alignment_amd import _lib
    _lib.lib()  # loud failure if the HIP library is missing
    return pkg


def gpu_value_and_grad(S, x, y, gamma, fused=False, checkpoint=False, low_memory=False):
    xd = x.to(DEV).requires_grad_(True)
    yd = y.to(DEV).requires_grad_(True)
    loss = S.soft_dtw(xd, yd, gamma, fused=fused, checkpoint=checkpoint, low_memory=low_memory)
    loss.mean().backward()
    torch.cuda.synchronize()
    return (loss.detach().cpu().double().numpy(), xd.grad.cpu().double().numpy(),
            yd.grad.cpu().double().numpy())


def assert_loss(l, l0, what=""):
    bad = np.abs(l - l0) > 1e-4 * np.abs(l0) + 1e-5
    assert not bad.any(), f"{what} loss mismatch: gpu {l[bad][:4]} oracle {l0[bad][:4]}"


def assert_grad(g, g0, what=""):
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    err = np.abs(g - g0)
    bad = err > 1e-5 + 1e-3 * np.abs(g0)
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{g.size} gradient elements "
                           f"out of tolerance, max err {err.max():.3e}")


def check_against_oracle(O, S, x, y, gamma, fused=False, pairs=None, what="", low_memory=False):
    l, gx, gy = gpu_value_and_grad(S, x, y, gamma, fused, low_memory=low_memory)
    assert np.isfinite(l).all() and np.isfinite(gx).all() and np.isfinite(gy).all()
    B = x.shape[0]
    idx = list(range(B)) if pairs is None else list(pairs)
    xs = x[idx].numpy()
    ys = y[idx].numpy()
    l0, gx0, gy0 = O.value_and_grad(xs, ys, gamma, np.full(len(idx), 1.0 / B),
                                    round_dist_f32=True)
    assert_loss(l[idx], l0, what)
    assert_grad(gx[idx], gx0, what + " dx")
    assert_grad(gy[idx], gy0, what + " dy")
    return l, gx, gy


# --- the distance kernel -----------------------------------------------------------------

@pytest.mark.parametrize("B,N,M,D", [(1, 1, 1, 1), (3, 37, 70, 5), (2, 64, 64, 64),
                                     (2, 129, 65, 128), (2, 200, 300, 3), (1, 33, 17, 256),
                                     (2, 16, 16, 1), (1, 70, 90, 7)])
def test_dist_matches_rounded_exact(O, S, B, N, M, D):
    x, y = pair_batch(B, N, M, D, seed=B + N + M + D)
    d = S.sqeuclidean(x.to(DEV), y.to(DEV)).cpu().double().numpy()
    ref = O.sqeuclid(x.numpy(), y.numpy(), round_f32=True)
    exact = O.sqeuclid(x.numpy(), y.numpy())
    assert (d >= 0).all()
    # fp64 accumulation then one rounding: equal to the nearest fp32 except
    # where the exact value sits within ~1e-13 of a rounding midpoint.
    diff = d != ref
    assert diff.mean() < 1e-4
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert (np.abs(d - exact) <= ulp).all()


# --- small and ragged shapes --------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True])
def test_tiny_config(O, S, fused):
    """B=2, N=M=16, D=1, gamma=1, mean loss."""
    x, y = pair_batch(2, 16, 16, 1, seed=0)
    check_against_oracle(O, S, x, y, 1.0, fused=fused, what="tiny")


@pytest.mark.parametrize("N,M", [(1, 1), (1, 9), (9, 1), (2, 2), (63, 65), (64, 64),
                                 (65, 63), (130, 257), (257, 130), (300, 300), (513, 77),
                                 (77, 513), (600, 333), (1100, 50), (5, 1500)])
@pytest.mark.parametrize("gamma", [1.0, 0.1])
@pytest.mark.parametrize("fused", [False, True])
def test_ragged_shapes(O, S, N, M, gamma, fused):
    x, y = pair_batch(3, N, M, 3, seed=N * 7 + M)
    check_against_oracle(O, S, x, y, gamma, fused=fused, what=f"{N}x{M} g={gamma}")


@pytest.mark.parametrize("N,M,D", [(150, 333, 240), (70, 130, 160), (90, 210, 136), (130, 77, 80)])
@pytest.mark.parametrize("fused", [False, True])
def test_ragged_wide_features(O, S, N, M, D, fused):
    """D above 128 on ragged lengths: the fused reverse's 64-column chain-rule
    helpers (three up to D = 192, four beyond; the last slice partial), each
    restaging its y rows for every one of the band's 16-column blocks."""
    x, y = pair_batch(3, N, M, D, seed=N + M + D)
    check_against_oracle(O, S, x, y, 0.5, fused=fused, what=f"{N}x{M} D={D}")


@pytest.mark.parametrize("seed", [1, 2])
def test_seeds(O, S, seed):
    x, y = pair_batch(4, 97, 111, 8, seed=seed)
    check_against_oracle(O, S, x, y, 0.5, what=f"seed {seed}")


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("B,N,M,D", [(2, 16, 16, 1), (32, 512, 512, 64), (32, 256, 256, 64)])
def test_seeds_on_workloads(O, S, seed, B, N, M, D):
    """Seeds 1 and 2 on the tiny, headline and feature-sweep (D=64) shapes,
    every pair against the oracle, unfused mode."""
    x, y = pair_batch(B, N, M, D, seed=seed)
    check_against_oracle(O, S, x, y, 1.0, what=f"{B}x{N}x{M} D={D} seed {seed}")


def test_alignment_matrix(O, S):
    x, y = pair_batch(2, 70, 45, 4, seed=21)
    l, E = S.alignment(x.to(DEV), y.to(DEV), 0.7)
    E = E.cpu().double().numpy()
    _, _, _, E0 = O.value_and_grad(x.numpy(), y.numpy(), 0.7, want_E=True)
    np.testing.assert_allclose(E, E0, rtol=1e-4, atol=1e-6)


# --- closed forms on the GPU ------------------------------------------------------------

@pytest.mark.parametrize("N,M", [(16, 16), (100, 100), (512, 512), (4096, 1000),
                                 (1024, 1024), (16, 9), (1, 7)])
def test_zero_distance_closed_form(S, N, M):
    vals = {(v["N"], v["M"]): v["log_delannoy"] for v in
            json.load(open(os.path.join(GOLD, "log_delannoy.json")))["values"]}
    x = torch.full((2, N, 5), 0.375, device=DEV)
    y = torch.full((2, M, 5), 0.375, device=DEV)
    for gamma in (1.0, 0.25):
        loss = S.soft_dtw(x, y, gamma).cpu().double().numpy()
        ref = -gamma * vals[(N, M)]
        np.testing.assert_allclose(loss, ref, rtol=1e-5)


@pytest.mark.parametrize("N,M", [(16, 16), (33, 20), (5, 60)])
def test_zero_distance_marginals(S, N, M):
    x = torch.full((1, N, 2), -1.5, device=DEV)
    y = torch.full((1, M, 2), -1.5, device=DEV)
    _, E = S.alignment(x, y, 1.0)
    np.testing.assert_allclose(E[0].cpu().double().numpy(), zero_dist_marginals(N, M),
                               rtol=2e-5, atol=1e-7)


# --- the workloads --------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True])
def test_headline_config(O, S, fused):
    """B=32, N=M=512, D=64, gamma=1, loss = batch mean; all pairs."""
    x, y = pair_batch(32, 512, 512, 64, seed=0)
    check_against_oracle(O, S, x, y, 1.0, fused=fused, what="headline")


@pytest.mark.parametrize("D", [1, 4, 16, 64, 128, 256])
@pytest.mark.parametrize("fused", [False, True])
def test_feature_sweep(O, S, D, fused):
    """B=32, N=M=256, D in {1,4,16,64,128,256}, gamma=1; all pairs."""
    x, y = pair_batch(32, 256, 256, D, seed=0)
    check_against_oracle(O, S, x, y, 1.0, fused=fused, what=f"D={D}")


@pytest.mark.parametrize("N,M", [(1024, 1024), (2048, 2048), (4096, 1000), (4096, 4096)])
@pytest.mark.parametrize("gamma", [1.0, 0.01])
@pytest.mark.parametrize("fused", [False, True])
def test_long_sequences(O, S, N, M, gamma, fused):
    """B=32, D=128 at full size on the GPU.  Sampling rule (the oracle would
    take minutes per pair at 4096^2): the oracle checks pairs 0 and 31
    elementwise, or pair 0 alone at 4096x4096; every one of the 32 pairs must
    be finite and have gradients summing to zero over both sequences
    (translation invariance of the squared distance), which holds at any
    size."""
    x, y = pair_batch(32, N, M, 128, seed=0)
    pairs = [0] if N * M > 5_000_000 else [0, 31]
    l, gx, gy = check_against_oracle(O, S, x, y, gamma, fused=fused, pairs=pairs,
                                     what=f"{N}x{M} g={gamma}")
    s = gx.sum(axis=1) + gy.sum(axis=1)
    scale = np.abs(gx).sum(axis=1) + np.abs(gy).sum(axis=1) + 1e-30
    assert (np.abs(s) <= 1e-4 * scale).all()


@pytest.mark.parametrize("N,M", [(2048, 2048), (4096, 1000)])
@pytest.mark.parametrize("gamma", [1.0, 0.01])
def test_long_sequences_low_memory(O, S, N, M, gamma):
    """The low-memory unfused mode at B=32, D=128 against the oracle (pairs
    0 and 31), with every pair finite and translation invariant."""
    x, y = pair_batch(32, N, M, 128, seed=0)
    l, gx, gy = check_against_oracle(O, S, x, y, gamma, pairs=[0, 31], low_memory=True,
                                     what=f"low-memory {N}x{M} g={gamma}")
    s = gx.sum(axis=1) + gy.sum(axis=1)
    scale = np.abs(gx).sum(axis=1) + np.abs(gy).sum(axis=1) + 1e-30
    assert (np.abs(s) <= 1e-4 * scale).all()


def test_barycenter_iterates(O, S):
    """10 block waves (100, 3), Adam lr 0.1, 100 iterations, gamma=1.  Both
    runs start from the same fp32 pointwise mean (computed on the CPU).  The
    first iterate's loss and gradient match the oracle to the usual
    tolerance; later iterates follow two independent Adam trajectories, so
    only the objective histories are compared, within 1e-3 relative (parity
    of the trajectory itself is unpinned: Adam amplifies rounding where
    gradients are near zero)."""
    X = block_waves(10, 100, 3, seed=0)
    z0 = X.mean(dim=0)
    f0, g0 = O.barycenter_objective_and_grad(z0.numpy(), X.numpy(), 1.0)
    Xd = X.to(DEV)
    z = z0.to(DEV).clone().requires_grad_(True)
    opt = torch.optim.Adam([z], lr=0.1)
    loss_fn = S.SoftDTW(gamma=1.0)
    hist = []
    for it in range(100):
        opt.zero_grad()
        loss = loss_fn(z.unsqueeze(0).expand_as(Xd), Xd).mean()
        loss.backward()
        hist.append(loss.item())
        if it == 0:
            assert abs(loss.item() - f0) <= 1e-4 * abs(f0) + 1e-5
            assert_grad(z.grad.cpu().double().numpy(), g0, "first iterate")
        opt.step()
    _, hist0 = O.barycenter(X.numpy(), 1.0, 100, 0.1, z0=z0.numpy())
    hist, hist0 = np.array(hist), np.array(hist0)
    assert np.abs(hist - hist0).max() <= 1e-3 * np.abs(hist0).max()
    assert hist[-1] < hist[0]


def test_barycenter_options_against_oracle(O, S):
    """Cosine annealing, gradient clipping and early stopping (README "Time
    Series Barycenters" key options, "Benchmarking"), on the block waves.
    The GPU loop and the oracle's fp64 loop take the same options; their
    objective histories agree to 1e-3 relative over the common length (the
    trajectories themselves are unpinned, as for plain Adam), and the GPU loop
    stops exactly where the oracle's rule fires on the GPU's own history."""
    X = block_waves(10, 100, 3, seed=0)
    z, hist = S.softdtw_barycenter(X.to(DEV), 1.0, 100, 0.1, cosine_annealing=True,
                                   grad_clip=1.0, early_stopping=True, patience=10,
                                   tol=1e-4, return_history=True)
    hist = hist.double().numpy()
    _, hist0 = O.barycenter(X.numpy(), 1.0, 100, 0.1, cosine=True, clip=1.0,
                            early_stopping=True, patience=10, tol=1e-4)
    k = O.stop_index(list(hist), 10, 1e-4)
    assert k is not None and len(hist) == k + 1 < 100
    n = min(len(hist), len(hist0))
    np.testing.assert_allclose(hist[:n], np.array(hist0[:n]), rtol=1e-3)
    assert torch.isfinite(z).all() and hist[-1] < hist[0]


def test_fused_auto_select(S):
    """fused=None / "auto" keeps the faster unfused mode while its workspace
    fits in half the free memory; D beyond fused mode's limit never selects
    it; a problem whose unfused workspace exceeds the free memory does."""
    assert S.choose_fused(None, 2, 50, 40, 3, DEV) is False
    assert S.choose_fused("auto", 2, 10, 10, 300, DEV) is False
    # unfused would take more than half the free memory: low-memory unfused
    # where that fits, else fused
    assert S.choose_mode(None, 32, 16384, 16384, 128, DEV) == 4
    assert S.choose_mode(None, 32, 20000, 20000, 128, DEV) == 1
    assert S.choose_fused(None, 32, 20000, 20000, 128, DEV) is True
    x, y = pair_batch(2, 50, 40, 3, seed=4)
    xd = x.to(DEV).requires_grad_(True)
    la = S.SoftDTW(gamma=0.5, fused="auto")(xd, y.to(DEV))
    lu = S.SoftDTW(gamma=0.5, fused=False)(xd, y.to(DEV))
    torch.testing.assert_close(la, lu, rtol=0, atol=0)


@pytest.mark.parametrize("fused,opts", [(False, {}),
                                        (False, {"cosine_annealing": True, "grad_clip": 1.0}),
                                        (True, {})])
def test_barycenter_loop_matches_autograd_loop(S, fused, opts):
    """softdtw_barycenter drives the C ABI directly on buffers it keeps for
    the whole loop; its objective history and final iterate equal those of
    the plain autograd loop (SoftDTW(...)(z expanded, X).mean().backward(),
    torch's fused Adam, clip_grad_norm_, the same options) started from the
    same iterate, to rounding (the gradient norm of the clipping is reduced
    by a different kernel there)."""
    X = block_waves(10, 100, 3, seed=2).to(DEV)
    T = 40
    z, hist = S.softdtw_barycenter(X, 1.0, T, 0.1, fused=fused, return_history=True, **opts)
    z0 = X.mean(dim=0).clone().requires_grad_(True)
    opt = torch.optim.Adam([z0], lr=0.1, fused=True)
    sched = (torch.optim.lr_scheduler.CosineAnnealingLR(opt, T_max=T)
             if opts.get("cosine_annealing") else None)
    loss_fn = S.SoftDTW(gamma=1.0, fused=fused)
    ref = []
    for _ in range(T):
        opt.zero_grad(set_to_none=True)
        loss = loss_fn(z0.unsqueeze(0).expand_as(X), X).mean()
        loss.backward()
        if "grad_clip" in opts:
            torch.nn.utils.clip_grad_norm_([z0], opts["grad_clip"])
        opt.step()
        if sched is not None:
            sched.step()
        ref.append(loss.item())
    assert len(hist) == T
    np.testing.assert_allclose(hist.double().numpy(), np.array(ref), rtol=1e-5)
    torch.testing.assert_close(z, z0.detach(), rtol=1e-4, atol=1e-5)


def test_barycenter_api(S):
    X = block_waves(10, 100, 3, seed=1).to(DEV)
    z, hist = S.softdtw_barycenter(X, gamma=1.0, max_iter=30, lr=0.1, return_history=True)
    assert z.shape == (100, 3) and torch.isfinite(z).all()
    assert hist[-1] < hist[0]


# --- fused mode against unfused mode ------------------------------------------------------

@pytest.mark.parametrize("N,M,D", [(70, 45, 4), (300, 260, 64), (129, 700, 100), (257, 64, 200),
                                   (150, 333, 240), (200, 150, 176), (65, 90, 20)])
def test_fused_matches_unfused(S, N, M, D):
    """Both modes see bit-identical distances and run the same recurrence, so
    the loss and the alignment matrix agree bitwise; gradients are summed in
    different orders (and dy through atomics in fused mode)."""
    x, y = pair_batch(3, N, M, D, seed=N + M + D)
    xd, yd = x.to(DEV), y.to(DEV)
    lu, Eu = S.alignment(xd, yd, 0.7, fused=False)
    lf, Ef = S.alignment(xd, yd, 0.7, fused=True)
    torch.testing.assert_close(lf, lu, rtol=0, atol=0)
    torch.testing.assert_close(Ef, Eu, rtol=0, atol=0)
    _, gxu, gyu = gpu_value_and_grad(S, x, y, 0.7, fused=False)
    _, gxf, gyf = gpu_value_and_grad(S, x, y, 0.7, fused=True)
    np.testing.assert_allclose(gxf, gxu, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(gyf, gyu, rtol=1e-4, atol=1e-6)


# --- checkpointed training against fused mode and the oracle -----------------------------

@pytest.mark.parametrize("B,N,M,D", [
    (2, 16, 16, 1),        # one band, one group
    (3, 300, 200, 5),      # 5 bands in groups of 3: two groups, ragged top
    (2, 256, 300, 64),     # 4 bands, groups of 2, N a multiple of 64
    (1, 513, 40, 3),       # 9 bands, groups of 3, one row in the top band
    (2, 1100, 70, 8),      # 18 bands, groups of 5
    (2, 130, 1100, 16),    # long M
    (2, 2100, 300, 32),    # 33 bands, groups of 6 (last group of 3)
    (2, 330, 150, 240),    # 6 bands, groups of 3, four 64-column chain-rule helpers
    (2, 200, 170, 176),    # 4 bands, groups of 2, three 64-column chain-rule helpers
    (2, 140, 260, 90),     # 3 bands, groups of 2, three 32-column chain-rule helpers
])
def test_checkpoint_matches_fused(S, B, N, M, D):
    """Checkpointed training recomputes the forward state group by group of
    rows from checkpoint rows: the same arithmetic on the same values as
    fused mode, so the loss, the alignment matrix and dx agree bitwise (dy
    is summed with atomics in both modes); a second backward on the same
    forward gives the same result."""
    x, y = pair_batch(B, N, M, D, seed=N + M + D + 7)
    xd, yd = x.to(DEV), y.to(DEV)
    lf, Ef = S.alignment(xd, yd, 0.8, fused=True)
    lc, Ec = S.alignment(xd, yd, 0.8, checkpoint=True)
    torch.testing.assert_close(lc, lf, rtol=0, atol=0)
    torch.testing.assert_close(Ec, Ef, rtol=0, atol=0)
    _, gxf, gyf = gpu_value_and_grad(S, x, y, 0.8, fused=True)
    xg = xd.clone().requires_grad_(True)
    yg = yd.clone().requires_grad_(True)
    loss = S.soft_dtw(xg, yg, 0.8, checkpoint=True).mean()
    gx1, gy1 = torch.autograd.grad(loss, (xg, yg), retain_graph=True)
    gx2, gy2 = torch.autograd.grad(loss, (xg, yg))
    np.testing.assert_array_equal(gx1.cpu().double().numpy(), gxf)
    torch.testing.assert_close(gx2, gx1, rtol=0, atol=0)
    np.testing.assert_allclose(gy1.cpu().double().numpy(), gyf, rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("B,N,M,D,gamma", [(3, 300, 200, 5, 1.0), (2, 700, 90, 4, 0.1)])
def test_checkpoint_against_oracle(O, S, B, N, M, D, gamma):
    x, y = pair_batch(B, N, M, D, seed=3 * N + M)
    l, gx, gy = gpu_value_and_grad(S, x, y, gamma, checkpoint=True)
    l0, gx0, gy0 = O.value_and_grad(x.numpy(), y.numpy(), gamma, np.full(B, 1.0 / B))
    assert_loss(l, l0, "checkpoint")
    assert_grad(gx, gx0, "checkpoint dx")
    assert_grad(gy, gy0, "checkpoint dy")


@pytest.mark.parametrize("gamma", [0.01])
def test_checkpoint_long_unequal_against_oracle(O, S, gamma):
    """Checkpointed training at the long unequal workload it exists for
    (B=32, N=4096, M=1000, D=128, gamma=0.01): the first and last pairs
    against the oracle, every pair finite with gradients summing to zero
    over both sequences (translation invariance)."""
    x, y = pair_batch(32, 4096, 1000, 128, seed=0)
    l, gx, gy = gpu_value_and_grad(S, x, y, gamma, checkpoint=True)
    assert np.isfinite(l).all() and np.isfinite(gx).all() and np.isfinite(gy).all()
    idx = [0, 31]
    l0, gx0, gy0 = O.value_and_grad(x[idx].numpy(), y[idx].numpy(), gamma,
                                    np.full(2, 1.0 / 32))
    assert_loss(l[idx], l0, "checkpoint 4096x1000")
    assert_grad(gx[idx], gx0, "checkpoint 4096x1000 dx")
    assert_grad(gy[idx], gy0, "checkpoint 4096x1000 dy")
    s = gx.sum(axis=1) + gy.sum(axis=1)
    scale = np.abs(gx).sum(axis=1) + np.abs(gy).sum(axis=1) + 1e-30
    assert (np.abs(s) <= 1e-4 * scale).all()


def test_checkpoint_workspace_is_smaller():
    from differentiable_series_alignment_amd import _lib as L
    fused = L.sdtw_workspace_bytes(32, 4096, 4096, 128, L.SDTW_MODE_FUSED)
    ck = L.sdtw_workspace_bytes(32, 4096, 4096, 128, L.SDTW_MODE_CHECKPOINT)
    assert 0 < ck * 5 < fused


def test_fused_rejects_large_D(S):
    from differentiable_series_alignment_amd import _lib
    assert _lib.sdtw_workspace_bytes(2, 10, 10, 300, _lib.SDTW_MODE_FUSED) == 0
    x, y = pair_batch(2, 10, 10, 300, seed=0)
    with pytest.raises(ValueError):
        S.soft_dtw(x.to(DEV), y.to(DEV), 1.0, fused=True)


# --- invariants (exact ones checked bitwise) ---------------------------------------------------

def test_power_of_two_scale_covariance_bitwise(S):
    x, y = pair_batch(4, 150, 170, 16, seed=3)
    l1, gx1, gy1 = gpu_value_and_grad(S, x, y, 0.5)
    l2, gx2, gy2 = gpu_value_and_grad(S, 2 * x, 2 * y, 2.0)
    np.testing.assert_array_equal(l2, 4 * l1)
    np.testing.assert_array_equal(gx2, 2 * gx1)
    np.testing.assert_array_equal(gy2, 2 * gy1)


def test_determinism_bitwise(S):
    x, y = pair_batch(8, 300, 280, 32, seed=4)
    a = gpu_value_and_grad(S, x, y, 0.3)
    b = gpu_value_and_grad(S, x, y, 0.3)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_symmetry_and_reversal(S):
    x, y = pair_batch(4, 120, 90, 6, seed=5)
    l, gx, gy = gpu_value_and_grad(S, x, y, 0.8)
    lt, gxt, gyt = gpu_value_and_grad(S, y, x, 0.8)
    lr_, _, _ = gpu_value_and_grad(S, x.flip(1), y.flip(1), 0.8)
    np.testing.assert_allclose(lt, l, rtol=1e-5)
    np.testing.assert_allclose(lr_, l, rtol=1e-5)
    assert_grad(gxt, gy, "symmetry")
    assert_grad(gyt, gx, "symmetry")


def test_normalized(O, S):
    x, y = pair_batch(3, 40, 40, 4, seed=6)
    f = S.SoftDTW(gamma=1.0, normalize=True)
    xd = x.to(DEV).requires_grad_(True)
    yd = y.to(DEV).requires_grad_(True)
    loss = f(xd, yd)
    loss.mean().backward()
    l0, gx0, gy0 = O.normalized_value_and_grad(x.numpy(), y.numpy(), 1.0)
    assert_loss(loss.detach().cpu().double().numpy(), l0, "normalized")
    assert_grad(xd.grad.cpu().double().numpy(), gx0, "normalized dx")
    assert_grad(yd.grad.cpu().double().numpy(), gy0, "normalized dy")
    self_loss = f(x.to(DEV), x.to(DEV))
    assert (self_loss == 0).all()


def test_retain_graph_twice(S):
    x, y = pair_batch(2, 50, 60, 3, seed=7)
    xd = x.to(DEV).requires_grad_(True)
    loss = S.soft_dtw(xd, y.to(DEV), 1.0).sum()
    loss.backward(retain_graph=True)
    g1 = xd.grad.clone()
    xd.grad = None
    loss.backward()
    torch.testing.assert_close(xd.grad, g1, rtol=0, atol=0)


def test_abi_backward_repeatable(S):
    """Through the C ABI: two backward calls on one unfused forward give
    bitwise the same dx, dy and E (the backward forms E from the sweep
    states and never reads the distances it overwrites); a backward with
    every output NULL is a successful no-op."""
    from differentiable_series_alignment_amd import _lib as L
    B, N, M, D = 3, 130, 97, 5
    x, y = pair_batch(B, N, M, D, seed=11)
    x, y = x.to(DEV), y.to(DEV)
    nb = L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_UNFUSED)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    loss = torch.empty(B, device=DEV)
    gl = torch.full((B,), 0.5, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, 1.0, L.SDTW_MODE_UNFUSED,
                           ws.data_ptr(), nb, loss.data_ptr(), s), "sdtw_forward")
    outs = []
    for _ in range(2):
        gx, gy = torch.empty_like(x), torch.empty_like(y)
        E = torch.empty(B, N, M, device=DEV)
        L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, 1.0,
                                L.SDTW_MODE_UNFUSED, ws.data_ptr(), nb, gl.data_ptr(),
                                gx.data_ptr(), gy.data_ptr(), E.data_ptr(), s), "sdtw_backward")
        outs.append((gx, gy, E))
    assert L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, 1.0, L.SDTW_MODE_UNFUSED,
                           ws.data_ptr(), nb, gl.data_ptr(), None, None, None, s) == L.SDTW_OK
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        torch.testing.assert_close(a, b, rtol=0, atol=0)
    assert torch.isfinite(outs[0][2]).all()


def _unfused_step(L, x, y, gamma, mode, want_e=True, backwards=1):
    """Unfused (mode 0) or low-memory unfused (mode 4) forward + backward(s)
    through the C ABI; returns the workspace size, loss and a list of (dx,
    dy, E) per backward."""
    B, N, D = x.shape
    M = y.shape[1]
    nb = L.sdtw_workspace_bytes(B, N, M, D, mode)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    loss = torch.empty(B, device=DEV)
    gl = torch.full((B,), 0.5, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode, ws.data_ptr(),
                           nb, loss.data_ptr(), s), "sdtw_forward")
    outs = []
    for _ in range(backwards):
        gx, gy = torch.empty_like(x), torch.empty_like(y)
        E = torch.empty(B, N, M, device=DEV) if want_e else None
        L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                                ws.data_ptr(), nb, gl.data_ptr(), gx.data_ptr(), gy.data_ptr(),
                                E.data_ptr() if want_e else None, s), "sdtw_backward")
        outs.append((gx, gy, E))
    assert L.sdtw_workspace_status(ws.data_ptr(), nb, B, N, M, D, mode, s) == L.SDTW_OK
    torch.cuda.synchronize()
    return nb, loss, outs


@pytest.mark.parametrize("B,N,M,D,gamma", [(3, 70, 45, 3, 1.0), (2, 300, 700, 5, 0.3),
                                           (3, 1100, 700, 5, 1.0), (2, 129, 600, 100, 0.1),
                                           (4, 512, 512, 64, 1.0)])
def test_low_memory_mode_matches_unfused(S, B, N, M, D, gamma):
    """The low-memory unfused mode (sweeps one after the other, the reverse
    sweep forming E over the distances in the backward) gives bitwise the
    loss, E and dx of the unfused mode, in a smaller workspace; dy too where
    both take the column pass (D > 64 or E requested), to rounding where the
    unfused mode sums the bands' shares instead.  A repeated backward reuses
    E."""
    from differentiable_series_alignment_amd import _lib as L
    x, y = (t.to(DEV) for t in pair_batch(B, N, M, D, seed=B + N + M))
    print(f"low-memory mode: {B}x{N}x{M}x{D}", flush=True)
    n1, l1, o1 = _unfused_step(L, x, y, gamma, 0)
    n2, l2, o2 = _unfused_step(L, x, y, gamma, 4, backwards=2)
    assert n2 < n1
    torch.testing.assert_close(l2, l1, rtol=0, atol=0)
    for gx, gy, E in o2:
        torch.testing.assert_close(E, o1[0][2], rtol=0, atol=0)
        torch.testing.assert_close(gx, o1[0][0], rtol=0, atol=0)
        torch.testing.assert_close(gy, o1[0][1], rtol=0, atol=0)   # E requested: column pass
    # without E the unfused mode takes the dy shares (D <= 64)
    _, _, o3 = _unfused_step(L, x, y, gamma, 0, want_e=False)
    _, _, o4 = _unfused_step(L, x, y, gamma, 4, want_e=False, backwards=2)
    for gx, gy, _ in o4:
        torch.testing.assert_close(gx, o3[0][0], rtol=0, atol=0)
        torch.testing.assert_close(gy, o3[0][1], rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("N", [64, 127, 192])
@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 33, 49, 63, 64, 65, 80, 81, 97])
def test_band_stride_edges_against_oracle(O, S, N, M):
    """The unfused arrays' bands lie sweep_steps(M) apart (M + 63 rounded up
    to 16), so the steps a sweep runs outside the grid's columns sit next to
    the neighbouring band's cells; M over every rounding residue, N whole and
    ragged (the reverse sweep's bands then straddle two bands of storage),
    checks that neither sweep, the E-forming reverse sweep nor the chain
    rule's E store writes over them.  Both unfused modes, E requested or
    not, against the oracle (loss, dx, dy, E)."""
    from differentiable_series_alignment_amd import _lib as L
    B, D, gamma = 3, 3, 0.5
    x, y = pair_batch(B, N, M, D, seed=N + M)
    l0, gx0, gy0, E0 = O.value_and_grad(x.numpy(), y.numpy(), gamma, np.full(B, 0.5),
                                        round_dist_f32=True, want_E=True)
    xd, yd = x.to(DEV), y.to(DEV)
    for mode in (L.SDTW_MODE_UNFUSED, L.SDTW_MODE_UNFUSED_LOWMEM):
        for want_e in (True, False):
            what = f"{B}x{N}x{M} mode {mode} E={want_e}"
            print(what, flush=True)
            _, loss, outs = _unfused_step(L, xd, yd, gamma, mode, want_e=want_e)
            gx, gy, E = outs[0]
            assert_loss(loss.cpu().double().numpy(), l0, what)
            assert_grad(gx.cpu().double().numpy(), gx0, what + " dx")
            assert_grad(gy.cpu().double().numpy(), gy0, what + " dy")
            if want_e:
                np.testing.assert_allclose(E.cpu().double().numpy(), E0, rtol=1e-4, atol=1e-6,
                                           err_msg=what + " E")


def test_low_memory_mode_launch_order(S):
    """Low-memory unfused: the forward call launches the distances and the
    forward sweep, the backward call the E-forming reverse sweep and the
    chain rule (row pass reading E, column pass)."""
    from differentiable_series_alignment_amd import _lib as L
    x, y = (t.to(DEV) for t in pair_batch(2, 100, 90, 8, seed=12))
    L.sdtw_timing(True)
    try:
        _unfused_step(L, x, y, 1.0, 4, want_e=False)
        recs = L.sdtw_timing_collect()
    finally:
        L.sdtw_timing(False)
    names = [n for n, _ in recs]
    assert names == ["dist_skew", "dp_forward", "dp_reverse_e", "chain_rows", "chain_cols"], names


def test_unfused_gradient_paths_agree(S):
    """Up to D = 64 dy comes from per-band shares made by the row pass; with
    the alignment matrix requested it comes from the column pass over E.
    Asking for dy alone gives bitwise the dy of a call that asks for both."""
    from differentiable_series_alignment_amd import _lib as L
    B, N, M, D = 3, 300, 170, 16
    x, y = pair_batch(B, N, M, D, seed=21)
    xd, yd = x.to(DEV), y.to(DEV)
    s = torch.cuda.current_stream().cuda_stream
    nb = L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_UNFUSED)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    loss = torch.empty(B, device=DEV)
    gl = torch.full((B,), 0.5, device=DEV)
    L.check(L.sdtw_forward(xd.data_ptr(), yd.data_ptr(), B, N, M, D, 0.9, 0, ws.data_ptr(),
                           nb, loss.data_ptr(), s), "sdtw_forward")
    outs = []
    for want_x, want_e in ((True, False), (False, False), (True, True)):
        gx = torch.zeros_like(xd)
        gy = torch.zeros_like(yd)
        E = torch.empty(B, N, M, device=DEV) if want_e else None
        L.check(L.sdtw_backward(xd.data_ptr(), yd.data_ptr(), B, N, M, D, 0.9, 0,
                                ws.data_ptr(), nb, gl.data_ptr(),
                                gx.data_ptr() if want_x else None, gy.data_ptr(),
                                E.data_ptr() if want_e else None, s), "sdtw_backward")
        outs.append((gx, gy))
    torch.testing.assert_close(outs[1][1], outs[0][1], rtol=0, atol=0)
    torch.testing.assert_close(outs[2][0], outs[0][0], rtol=0, atol=0)
    torch.testing.assert_close(outs[2][1], outs[0][1], rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("D,chain", [(8, ["chain_rows", "chain_gy"]),
                                     (100, ["chain_rows", "chain_cols"])])
def test_launch_timing_records_each_kernel(S, D, chain):
    """sdtw_timing brackets every launch of a forward+backward with events on
    the call's stream and reports them by name, in launch order.  Up to
    D = 64 the row pass also makes the bands' shares of dy, which a short
    pass adds up; beyond, a column pass reads E."""
    from differentiable_series_alignment_amd import _lib as L
    x, y = pair_batch(2, 100, 90, D, seed=12)
    xd = x.to(DEV).requires_grad_(True)
    yd = y.to(DEV).requires_grad_(True)
    L.sdtw_timing(True)
    try:
        S.soft_dtw(xd, yd, 1.0).sum().backward()
        recs = L.sdtw_timing_collect()
    finally:
        L.sdtw_timing(False)
    names = [n for n, _ in recs]
    assert names == ["dist_skew", "dp_both"] + chain, names
    assert all(t > 0 for _, t in recs)


@pytest.mark.parametrize("B,N,M,D", [
    (2, 16, 16, 1), (3, 70, 45, 3),                       # whole rows (M <= 512)
    (3, 1100, 700, 5), (2, 300, 2000, 4), (1, 64, 5000, 2), (4, 130, 513, 8),  # rings
    (40, 500, 600, 3),                                    # whole rows, band-major
    (9, 2048, 8192, 2),                                   # rings, more bands than CUs
    (2, 300, 700, 100), (3, 200, 300, 160),               # D > 64: six distance helpers
])
def test_inference_mode_matches_training_loss(S, B, N, M, D):
    """The inference mode (no state kept; rows handed between bands whole
    or through 512-column rings) returns bitwise the training forward's
    loss, through the C ABI; without autograd the Python layer uses it."""
    from differentiable_series_alignment_amd import _lib as L
    x, y = pair_batch(B, N, M, D, seed=B + N + M + D)
    x, y = x.to(DEV), y.to(DEV)
    s = torch.cuda.current_stream().cuda_stream
    out = {}
    for mode in (L.SDTW_MODE_UNFUSED, L.SDTW_MODE_INFERENCE):
        nb = L.sdtw_workspace_bytes(B, N, M, D, mode)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        loss = torch.empty(B, device=DEV)
        for _ in range(2):   # the second call finds the control words it left
            L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, 0.6, mode,
                                   ws.data_ptr(), nb, loss.data_ptr(), s), "sdtw_forward")
        out[mode] = loss
    torch.testing.assert_close(out[L.SDTW_MODE_INFERENCE], out[L.SDTW_MODE_UNFUSED],
                               rtol=0, atol=0)
    with torch.no_grad():
        torch.testing.assert_close(S.soft_dtw(x, y, 0.6), out[L.SDTW_MODE_UNFUSED],
                                   rtol=0, atol=0)


def inference_loss(S, x, y, gamma):
    """Loss through the C ABI in inference mode (no state kept)."""
    from differentiable_series_alignment_amd import _lib as L
    B, N, D = x.shape
    M = y.shape[1]
    xd, yd = x.to(DEV), y.to(DEV)
    nb = L.sdtw_workspace_bytes(B, N, M, D, L.SDTW_MODE_INFERENCE)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    loss = torch.empty(B, device=DEV)
    L.check(L.sdtw_forward(xd.data_ptr(), yd.data_ptr(), B, N, M, D, gamma,
                           L.SDTW_MODE_INFERENCE, ws.data_ptr(), nb, loss.data_ptr(),
                           torch.cuda.current_stream().cuda_stream), "sdtw_forward")
    torch.cuda.synchronize()
    return loss.cpu().double().numpy()


@pytest.mark.parametrize("B,N,M,D,pairs", [
    (3, 70, 45, 3, None),            # whole hand-off rows
    (3, 1100, 700, 5, None),         # 512-column rings
    (9, 2048, 8192, 2, [0, 8]),      # rings, more bands than the GPU has CUs
])
@pytest.mark.parametrize("gamma", [1.0, 0.1])
def test_inference_mode_against_oracle(O, S, B, N, M, D, pairs, gamma):
    """The loss-only inference mode (the README's "When to Use Each Mode":
    speed-critical inference) against the oracle's loss on random N(0,1)
    inputs, for whole-row and ring hand-off; the largest shape checks the
    first and last pairs."""
    x, y = pair_batch(B, N, M, D, seed=B * 13 + N + M + D)
    l = inference_loss(S, x, y, gamma)
    assert np.isfinite(l).all()
    idx = list(range(B)) if pairs is None else pairs
    l0, _, _ = O.value_and_grad(x[idx].numpy(), y[idx].numpy(), gamma)
    assert_loss(l[idx], l0, f"inference {B}x{N}x{M} g={gamma}")


def test_normalized_is_one_batch(S):
    """SoftDTW(normalize=True) runs its three terms as one batch of 3B pairs."""
    from differentiable_series_alignment_amd import _lib as L
    x, y = pair_batch(3, 40, 40, 4, seed=13)
    xd = x.to(DEV).requires_grad_(True)
    L.sdtw_timing(True)
    try:
        S.SoftDTW(gamma=1.0, normalize=True)(xd, y.to(DEV)).sum().backward()
        names = [n for n, _ in L.sdtw_timing_collect()]
    finally:
        L.sdtw_timing(False)
    assert names.count("dp_both") == 1, names


def test_small_gamma_finite(S):
    x, y = pair_batch(4, 700, 650, 32, seed=8)
    l, gx, gy = gpu_value_and_grad(S, x, y, 0.01)
    assert np.isfinite(l).all() and np.isfinite(gx).all() and np.isfinite(gy).all()


@pytest.mark.parametrize("mode", [0, 1, 3])
def test_workspace_contents_do_not_matter(S, mode):
    """Rows handed between workgroups carry their own validity and every
    forward sets them: a workspace left holding zeros (which read as valid
    values) or all-ones bytes (NaNs) gives bitwise the same loss and dx, and
    a second backward on one forward repeats the first (each sweep leaves
    the rows as it found them)."""
    from differentiable_series_alignment_amd import _lib as L
    B, N, M, D = 2, 300, 150, 8      # 5 bands: two segments unfused, five fused
    x, y = pair_batch(B, N, M, D, seed=5)
    x, y = x.to(DEV), y.to(DEV)
    nb = L.sdtw_workspace_bytes(B, N, M, D, mode)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    gl = torch.full((B,), 0.5, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    runs = []
    for fill in (0, 255):
        ws.fill_(fill)
        loss = torch.empty(B, device=DEV)
        L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, 1.0, mode,
                               ws.data_ptr(), nb, loss.data_ptr(), s), "sdtw_forward")
        grads = []
        for _ in range(2):
            gx, gy = torch.empty_like(x), torch.empty_like(y)
            L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, 1.0, mode,
                                    ws.data_ptr(), nb, gl.data_ptr(), gx.data_ptr(),
                                    gy.data_ptr(), None, s), "sdtw_backward")
            grads.append((gx, gy))
        torch.cuda.synchronize()
        assert torch.isfinite(loss).all()
        torch.testing.assert_close(grads[1][0], grads[0][0], rtol=0, atol=0)
        torch.testing.assert_close(grads[1][1], grads[0][1], rtol=1e-5, atol=1e-7)
        runs.append((loss, grads[0]))
    torch.testing.assert_close(runs[1][0], runs[0][0], rtol=0, atol=0)
    torch.testing.assert_close(runs[1][1][0], runs[0][1][0], rtol=0, atol=0)
    torch.testing.assert_close(runs[1][1][1], runs[0][1][1], rtol=1e-5, atol=1e-7)


def test_inference_workspace_contents_do_not_matter(S):
    """The loss-only forward with whole hand-off rows: a workspace holding
    zeros or all-ones bytes gives bitwise the same loss, equal to the
    training forward's."""
    from differentiable_series_alignment_amd import _lib as L
    B, N, M, D = 2, 300, 150, 8
    x, y = pair_batch(B, N, M, D, seed=6)
    x, y = x.to(DEV), y.to(DEV)
    s = torch.cuda.current_stream().cuda_stream
    losses = []
    for mode, fill in ((L.SDTW_MODE_INFERENCE, 0), (L.SDTW_MODE_INFERENCE, 255),
                       (L.SDTW_MODE_UNFUSED, 0)):
        nb = L.sdtw_workspace_bytes(B, N, M, D, mode)
        ws = torch.full((nb,), fill, dtype=torch.uint8, device=DEV)
        loss = torch.empty(B, device=DEV)
        L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, 1.0, mode,
                               ws.data_ptr(), nb, loss.data_ptr(), s), "sdtw_forward")
        torch.cuda.synchronize()
        losses.append(loss)
    torch.testing.assert_close(losses[1], losses[0], rtol=0, atol=0)
    torch.testing.assert_close(losses[2], losses[0], rtol=0, atol=0)

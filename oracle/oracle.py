"""Python face of the fp64 Soft-DTW oracle.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  Nothing here is imported by the product
package, and nothing here imports it.

The arithmetic lives in ``sdtw_oracle.c`` (fp64, libm); this module marshals
numpy arrays and composes the C entry points into the pages' user-level
operations:

* ``value_and_grad``: the Soft-DTW loss per pair and its gradients w.r.t. x
  and y ("Usage" of the README "SoftDTW-CUDA (PyTorch + Numba)": a (B,) loss
  that is averaged and back-propagated).
* ``normalized_value_and_grad``: SoftDTW(x,y) - (SoftDTW(x,x) + SoftDTW(y,y))/2
  (README section "Normalization"; equal shapes only).
* ``barycenter``: Adam on the mean Soft-DTW between a free sequence and the
  given ones (README "Time Series Barycenters"; review page, section
  "Proposed method": barycenters by Adam), with the README's optional
  cosine annealing, gradient clipping and early stopping ("Benchmarking").

Readings taken where the pages are silent are listed with each function.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsdtw_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def lib():
    """Load (building once with gcc if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _b  # local build helper, gcc only
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_sqeuclid.argtypes = [_f32p, _f32p, _i64, _i64, _i64, _i64, _f64p]
        L.oracle_sqeuclid.restype = None
        L.oracle_sdtw_forward.argtypes = [_f64p, _i64, _i64, _i64, ctypes.c_double,
                                          ctypes.c_void_p, _f64p]
        L.oracle_sdtw_forward.restype = ctypes.c_int
        L.oracle_sdtw_backward.argtypes = [_f64p, _f64p, _i64, _i64, _i64,
                                           ctypes.c_double, _f64p]
        L.oracle_sdtw_backward.restype = ctypes.c_int
        L.oracle_sdtw_backward_local.argtypes = [_f64p, _i64, _i64, _i64,
                                                 ctypes.c_double, _f64p]
        L.oracle_sdtw_backward_local.restype = ctypes.c_int
        L.oracle_sqeuclid_vjp.argtypes = [_f32p, _f32p, _f64p, _f64p, _i64, _i64,
                                          _i64, _i64, _f64p, _f64p]
        L.oracle_sqeuclid_vjp.restype = None
        L.oracle_sdtw_value_and_grad.argtypes = [
            _f32p, _f32p, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int,
            _f64p, _f64p, _f64p, _f64p, ctypes.c_void_p]
        L.oracle_sdtw_value_and_grad.restype = ctypes.c_int
        L.oracle_dtw.argtypes = [_f64p, _i64, _i64, _i64, _f64p]
        L.oracle_dtw.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle inputs are the fp32 sequences themselves")
    return np.ascontiguousarray(a)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _check(rc: int):
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP regions from now on (timing)."""
    lib().oracle_set_num_threads(int(n))


def sqeuclid(x, y, round_f32: bool = False) -> np.ndarray:
    """Dist[b,i,j] = sum_d (x[b,i,d] - y[b,j,d])^2 in fp64 (direct form).

    With ``round_f32`` the exact value is rounded to the nearest fp32, i.e.
    the content of an fp32 (B,N,M) distance tensor (reading: the unfused
    mode's materialised tensor has the inputs' dtype)."""
    x, y = _f32(x), _f32(y)
    B, N, D = x.shape
    B2, M, D2 = y.shape
    assert B == B2 and D == D2
    out = np.empty((B, N, M), dtype=np.float64)
    lib().oracle_sqeuclid(x, y, B, N, M, D, out)
    if round_f32:
        out = out.astype(np.float32).astype(np.float64)
    return out


def forward(dist, gamma: float, keep_R: bool = True):
    """Soft-DTW forward on a (B,N,M) fp64 Dist. Returns (loss[B], R or None);
    R is (B, N+1, M+1) with the +inf / 0 boundary row and column."""
    dist = _f64(dist)
    B, N, M = dist.shape
    loss = np.empty(B, dtype=np.float64)
    R = np.empty((B, N + 1, M + 1), dtype=np.float64) if keep_R else None
    rp = R.ctypes.data_as(ctypes.c_void_p) if keep_R else None
    _check(lib().oracle_sdtw_forward(dist, B, N, M, float(gamma), rp, loss))
    return loss, R


def backward(dist, R, gamma: float) -> np.ndarray:
    """Alignment matrix E = dLoss/dDist by the log-space (logsumexp) backward
    with the exponential applied at the end."""
    dist, R = _f64(dist), _f64(R)
    B, N, M = dist.shape
    E = np.empty((B, N, M), dtype=np.float64)
    _check(lib().oracle_sdtw_backward(dist, R, B, N, M, float(gamma), E))
    return E


def backward_local(R, gamma: float) -> np.ndarray:
    """Same E through locally re-derived softmin weights (cross-check only)."""
    R = _f64(R)
    B, N1, M1 = R.shape
    E = np.empty((B, N1 - 1, M1 - 1), dtype=np.float64)
    _check(lib().oracle_sdtw_backward_local(R, B, N1 - 1, M1 - 1, float(gamma), E))
    return E


def sqeuclid_vjp(x, y, E, grad_loss):
    """Chain rule through Dist: (gx, gy) in fp64 for per-pair upstream grads."""
    x, y, E = _f32(x), _f32(y), _f64(E)
    B, N, D = x.shape
    M = y.shape[1]
    gl = _f64(np.broadcast_to(np.asarray(grad_loss, dtype=np.float64), (B,)))
    gx = np.empty((B, N, D), dtype=np.float64)
    gy = np.empty((B, M, D), dtype=np.float64)
    lib().oracle_sqeuclid_vjp(x, y, E, gl, B, N, M, D, gx, gy)
    return gx, gy


def value_and_grad(x, y, gamma: float, grad_loss=None, round_dist_f32: bool = True,
                   want_E: bool = False):
    """Loss[B] and (gx, gy) for upstream gradients ``grad_loss`` (default: the
    batch mean, 1/B each, as in ``loss_fn(x, y).mean().backward()``).

    Memory is bounded by per-thread scratch, so full-size pairs are fine.
    ``round_dist_f32`` selects the reading of Dist (see ``sqeuclid``)."""
    x, y = _f32(x), _f32(y)
    B, N, D = x.shape
    M = y.shape[1]
    if grad_loss is None:
        grad_loss = np.full(B, 1.0 / B)
    gl = _f64(np.broadcast_to(np.asarray(grad_loss, dtype=np.float64), (B,)))
    loss = np.empty(B, dtype=np.float64)
    gx = np.empty((B, N, D), dtype=np.float64)
    gy = np.empty((B, M, D), dtype=np.float64)
    E = np.empty((B, N, M), dtype=np.float64) if want_E else None
    ep = E.ctypes.data_as(ctypes.c_void_p) if want_E else None
    _check(lib().oracle_sdtw_value_and_grad(x, y, B, N, M, D, float(gamma),
                                            int(bool(round_dist_f32)), gl, loss,
                                            gx, gy, ep))
    if want_E:
        return loss, gx, gy, E
    return loss, gx, gy


def dtw(dist) -> np.ndarray:
    """Hard DTW (min recurrence) per pair."""
    dist = _f64(dist)
    B, N, M = dist.shape
    out = np.empty(B, dtype=np.float64)
    _check(lib().oracle_dtw(dist, B, N, M, out))
    return out


def normalized_value_and_grad(x, y, gamma: float, grad_loss=None,
                              round_dist_f32: bool = True):
    """SoftDTW(x,y) - (SoftDTW(x,x) + SoftDTW(y,y))/2 and its gradients.

    The pages require x.shape == y.shape.  The gradient of SoftDTW(x,x)
    w.r.t. x is the sum of its two argument gradients."""
    x, y = _f32(x), _f32(y)
    if x.shape != y.shape:
        raise ValueError("normalized Soft-DTW needs x.shape == y.shape")
    B = x.shape[0]
    if grad_loss is None:
        grad_loss = np.full(B, 1.0 / B)
    gl = np.broadcast_to(np.asarray(grad_loss, dtype=np.float64), (B,))
    lxy, gxy_x, gxy_y = value_and_grad(x, y, gamma, gl, round_dist_f32)
    lxx, gxx_a, gxx_b = value_and_grad(x, x, gamma, -0.5 * gl, round_dist_f32)
    lyy, gyy_a, gyy_b = value_and_grad(y, y, gamma, -0.5 * gl, round_dist_f32)
    loss = lxy - 0.5 * (lxx + lyy)
    return loss, gxy_x + gxx_a + gxx_b, gxy_y + gyy_a + gyy_b


def adam_init(shape):
    return {"t": 0, "m": np.zeros(shape), "v": np.zeros(shape)}


def adam_step(p, grad, state, lr, betas=(0.9, 0.999), eps=1e-8):
    """Textbook Adam (Kingma & Ba) with bias correction, fp64, in place.

    Reading: the pages give only the learning rate; betas and eps are the
    usual defaults."""
    b1, b2 = betas
    state["t"] += 1
    t = state["t"]
    state["m"] = b1 * state["m"] + (1.0 - b1) * grad
    state["v"] = b2 * state["v"] + (1.0 - b2) * grad * grad
    mhat = state["m"] / (1.0 - b1 ** t)
    vhat = state["v"] / (1.0 - b2 ** t)
    p -= lr * mhat / (np.sqrt(vhat) + eps)
    return p


def barycenter_objective_and_grad(z, X, gamma: float, round_dist_f32: bool = True):
    """f(z) = mean_k SoftDTW(z, X_k) and df/dz for z (T,D) fp32-representable."""
    X = _f32(X)
    K = X.shape[0]
    zb = np.ascontiguousarray(np.broadcast_to(np.asarray(z, dtype=np.float32),
                                              (K,) + tuple(np.shape(z))))
    loss, gz, _ = value_and_grad(zb, X, gamma, np.full(K, 1.0 / K), round_dist_f32)
    return float(loss.mean()), gz.sum(axis=0)


def cosine_lr(lr: float, t: int, T: int) -> float:
    """Learning rate of iteration t (0-based) of T under cosine annealing to
    zero: lr * (1 + cos(pi t / T)) / 2 (Loshchilov & Hutter's SGDR schedule
    without restarts).  The README ("Benchmarking") names cosine annealing
    for the barycenter loop without parameters; reading: over max_iter
    iterations, down to 0."""
    return 0.5 * lr * (1.0 + math.cos(math.pi * t / T))


def clip_by_norm(g, c: float):
    """Gradient clipping by global L2 norm: g * min(1, c / (|g| + 1e-6))
    (the README's "Benchmarking" names gradient clipping without details;
    reading: norm clipping with the customary 1e-6 guard)."""
    g = np.asarray(g, dtype=np.float64)
    n = math.sqrt(float(np.sum(g * g)))
    return g * min(1.0, c / (n + 1e-6))


def stop_index(history, patience: int, tol: float):
    """First iteration index after which the early-stopping rule fires, or
    None.  Reading (the README's "Time Series Barycenters" only says early
    stopping detects convergence): a value below best - tol*|best| is an
    improvement and resets the count; any other value is a stall; the rule
    fires at the patience-th stall in a row.  The first value is always an
    improvement."""
    best = None
    stalls = 0
    for i, f in enumerate(history):
        if best is None or f < best - tol * abs(best):
            best = f
            stalls = 0
        else:
            stalls += 1
            if stalls == patience:
                return i
    return None


def barycenter(X, gamma: float = 1.0, max_iter: int = 100, lr: float = 0.1,
               round_dist_f32: bool = True, z0=None, cosine: bool = False,
               clip=None, early_stopping: bool = False, patience: int = 10,
               tol: float = 1e-4):
    """Adam on mean_k SoftDTW(z, X_k), z initialised to the pointwise mean
    (or to ``z0`` when given).  Each iteration evaluates the objective and
    its gradient at the current iterate, clips the gradient (``clip``),
    takes an Adam step at the iteration's learning rate (``cosine``), and
    then applies the early-stopping rule to the objectives seen so far.

    Reading: the iterate is kept in fp32 between steps (the sequences are
    fp32 and the objective is evaluated on fp32 inputs); the Adam update
    itself is fp64.  Returns (z, objective history)."""
    X = _f32(X)
    z = (X.astype(np.float64).mean(axis=0) if z0 is None
         else np.asarray(z0, dtype=np.float64).copy())
    st = adam_init(z.shape)
    hist = []
    for t in range(max_iter):
        zf = z.astype(np.float32)
        f, g = barycenter_objective_and_grad(zf, X, gamma, round_dist_f32)
        hist.append(f)
        if clip is not None:
            g = clip_by_norm(g, clip)
        z = zf.astype(np.float64)
        adam_step(z, g, st, cosine_lr(lr, t, max_iter) if cosine else lr)
        if early_stopping and stop_index(hist, patience, tol) is not None:
            break
    return z.astype(np.float32), hist

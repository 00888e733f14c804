"""Model of the split-integer distance arithmetic of the HIP library, written
from its specification for the tests (it is neither the oracle nor shared
with the HIP sources): per-row power-of-two scaling, six balanced base-256
digits per element, level sums of digit products, and the fp64 combination.

Specification (the library's distance kernels follow it operation by
operation, so their fp32 output equals this model's bit for bit):

* Row scale.  a = max_d |v_d| (fp32).  a = 0 gives e = 0; otherwise e is the
  integer with 2^(e-3) <= a < 2^(e-2), so |v_d| 2^-e < 1/4.
* Integer.  Z_d = rint(v_d 2^(48-e)) (round half to even), |Z_d| < 2^46.
  Computed as h = v 2^(24-e), hi = rint(h), lo = rint((h - hi) 2^24), which
  is exact in fp32 and gives Z = hi 2^24 + lo.
* Digits.  U = Z + 0x808080808080 lies in [0, 2^48); its base-256 digits
  u_1 (most significant) .. u_6 give g_k = u_k - 128 in [-128, 127] and
  Z = sum_k g_k 256^(6-k).
* Levels.  For each block of 64 features, A_L = sum_d sum_{i+j=L} g_i(x_d)
  g_j(y_d) for L = 2..7 (21 digit pairs; pairs with i+j >= 8 are dropped),
  and C23 = 256 A_2 + A_3, C45 = 256 A_4 + A_5, C67 = 256 A_6 + A_7, each
  below 2^31 in magnitude (so exact in int32).
* Combination (fp64).  Per block t_b = (C67 2^-16 + C45) 2^-16 + C23, and
  t = t_0 + t_1 + ... over the blocks in order; x.y ~ 2^(ex+ey-24) t.
  Norms n = sum_d v_d^2 in fp64, d in order; s = nx + ny;
  v = s - 2^(ex+ey-23) t.  Every product so far is by a power of two, so
  multiply-then-add and fused multiply-add give the same bits.
* Correct rounding (Ziv's test).  |v - Dist| <= eps with
  eps = s c2 + 2^(ex+ey) c1 (a product then a sum, each rounded once),
  c1 = 2.02 D (6.05 + (nb + 1)/64) 2^-50, c2 = (1.02 D + 6) 2^-53, nb the
  number of 64-feature blocks (bound_constants derives them).  If
  fp32(max(0, v - eps)) == fp32(max(0, v + eps)) that value is the exact
  distance rounded once to fp32; otherwise the distance is summed directly,
  sum_d (x_d - y_d)^2 in fp64 with d in order, and rounded to fp32.
"""
from __future__ import annotations

import numpy as np

OFFSET = 0x808080808080


def row_exponent(v: np.ndarray) -> np.ndarray:
    """e per row of v [..., D] (fp32): 2^(e-3) <= max|v| < 2^(e-2)."""
    a = np.max(np.abs(v.astype(np.float32)), axis=-1)
    m, E = np.frexp(a.astype(np.float64))        # a = m 2^E, m in [0.5, 1)
    e = (E + 2).astype(np.int64)
    return np.where(a == 0, 0, e)


def integers(v: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Z = rint(v 2^(48-e)) per element, by the fp32 two-step route."""
    v = v.astype(np.float32)
    sc = np.ldexp(np.float32(1), (24 - e)[..., None]).astype(np.float32)
    h = (v * sc).astype(np.float32)
    hi = np.rint(h).astype(np.float32)
    r = (h - hi).astype(np.float32)
    lo = np.rint((r * np.float32(2.0 ** 24)).astype(np.float32))
    return hi.astype(np.int64) * (1 << 24) + lo.astype(np.int64)


def digits(Z: np.ndarray) -> np.ndarray:
    """Balanced base-256 digits [..., 6] (most significant first)."""
    U = Z + OFFSET
    assert (U >= 0).all() and (U < (1 << 48)).all()
    out = np.empty(Z.shape + (6,), dtype=np.int64)
    for k in range(6):
        out[..., 5 - k] = ((U >> (8 * k)) & 0xFF) - 128
    return out


def levels(gx: np.ndarray, gy: np.ndarray) -> np.ndarray:
    """A_L, L = 2..7, for one block: gx [N, d, 6], gy [M, d, 6] -> [N, M, 6]."""
    N, M = gx.shape[0], gy.shape[0]
    A = np.zeros((N, M, 6), dtype=np.int64)
    for i in range(1, 7):
        for j in range(1, 7):
            L = i + j
            if L <= 7:
                A[:, :, L - 2] += gx[:, :, i - 1] @ gy[:, :, j - 1].T
    return A


def bound_constants(D: int):
    """(c1, c2) of the error bound eps = s c2 + 2^(ex+ey) c1 on v.

    Per feature the product of the scaled values X Y (|X|, |Y| < 1/4)
    differs from its kept digit pairs by at most 2^-50 (rounding of the
    integers: (|X| + |Y|) 2^-49 + 2^-98) plus 5.02 2^-50 (the dropped
    pairs, i + j >= 8: at most 5, 4, 3, 2, 1 pairs of |g_i g_j| <= 2^14 at
    weights 2^-64, 2^-72, ...), and the fp64 combination adds at most
    (nb + 1) 2^-56 per feature; doubled for 2 x.y, times 1.01 for the
    rounding of eps itself.  The norms carry at most 1.01 D 2^-53 of s,
    the sum s and v one rounding each, and the bracket v -/+ eps two more
    of |v| <= 2 s: (1.02 D + 6) 2^-53 covers them."""
    nb = (D + 63) // 64
    c1 = 2.02 * D * (6.05 + (nb + 1) / 64.0) * 2.0 ** -50
    c2 = (1.02 * D + 6.0) * 2.0 ** -53
    return c1, c2


def sqdist(x: np.ndarray, y: np.ndarray, return_parts: bool = False):
    """Dist [N, M] (fp32) of one pair x [N, D], y [M, D] by the specification."""
    x = np.asarray(x, dtype=np.float32)
    y = np.asarray(y, dtype=np.float32)
    D = x.shape[1]
    ex, ey = row_exponent(x), row_exponent(y)
    gx, gy = digits(integers(x, ex)), digits(integers(y, ey))
    t = np.zeros((x.shape[0], y.shape[0]), dtype=np.float64)
    cmax = 0
    for d0 in range(0, D, 64):
        A = levels(gx[:, d0:d0 + 64], gy[:, d0:d0 + 64])
        C23 = 256 * A[..., 0] + A[..., 1]
        C45 = 256 * A[..., 2] + A[..., 3]
        C67 = 256 * A[..., 4] + A[..., 5]
        cmax = max(cmax, int(np.abs(np.stack([C23, C45, C67])).max()))
        tb = (C67.astype(np.float64) * 2.0 ** -16 + C45.astype(np.float64)) * 2.0 ** -16 \
            + C23.astype(np.float64)
        t = t + tb
    nx = np.zeros(x.shape[0])
    for d in range(D):
        nx = nx + x[:, d].astype(np.float64) ** 2
    ny = np.zeros(y.shape[0])
    for d in range(D):
        ny = ny + y[:, d].astype(np.float64) ** 2
    exy = (ex[:, None] + ey[None, :]).astype(np.int64)
    s = nx[:, None] + ny[None, :]
    v = s + (-np.ldexp(1.0, exy - 23)) * t
    c1, c2 = bound_constants(D)
    eps = s * c2 + np.ldexp(c1, exy)
    lo = np.maximum(v - eps, 0.0).astype(np.float32)
    hi = np.maximum(v + eps, 0.0).astype(np.float32)
    amb = lo != hi
    out = lo.copy()
    if amb.any():
        ii, jj = np.nonzero(amb)
        acc = np.zeros(len(ii))
        for d in range(D):
            diff = x[ii, d].astype(np.float64) - y[jj, d].astype(np.float64)
            acc = acc + diff * diff
        out[ii, jj] = acc.astype(np.float32)
    if return_parts:
        return out, dict(ex=ex, ey=ey, gx=gx, gy=gy, t=t, nx=nx, ny=ny, cmax=cmax, v=v,
                         eps=eps, ambiguous=amb)
    return out

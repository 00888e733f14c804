"""Independent references used to pin the oracle (tests only).

Nothing here shares code with ``oracle/``: brute force over every monotone
alignment path, exact Delannoy-number closed forms, and small helpers.
"""
from __future__ import annotations

import math
from fractions import Fraction
from functools import lru_cache

import numpy as np


def monotone_paths(N: int, M: int):
    """All alignment paths from (0,0) to (N-1,M-1) with steps (1,0), (0,1),
    (1,1); each path is a tuple of cells."""
    out = []

    def rec(i, j, acc):
        if i == N - 1 and j == M - 1:
            out.append(tuple(acc))
            return
        for di, dj in ((1, 0), (0, 1), (1, 1)):
            a, b = i + di, j + dj
            if a < N and b < M:
                acc.append((a, b))
                rec(a, b, acc)
                acc.pop()

    rec(0, 0, [(0, 0)])
    return out


def brute_force(dist: np.ndarray, gamma: float):
    """Soft-DTW as a soft minimum over all paths, and its path marginals:
    value = -gamma * log sum_p exp(-cost_p / gamma),
    E[i,j] = sum over paths through (i,j) of softmax(-cost / gamma)_p."""
    N, M = dist.shape
    paths = monotone_paths(N, M)
    costs = np.array([sum(dist[i, j] for i, j in p) for p in paths])
    z = -costs / gamma
    zmax = z.max()
    w = np.exp(z - zmax)
    total = w.sum()
    value = -gamma * (zmax + math.log(total))
    E = np.zeros((N, M))
    for p, wp in zip(paths, w / total):
        for i, j in p:
            E[i, j] += wp
    return value, E, costs.min(), len(paths)


@lru_cache(maxsize=None)
def delannoy(m: int, n: int) -> int:
    """Number of lattice paths from (0,0) to (m,n) with steps E, N, NE."""
    if m == 0 or n == 0:
        return 1
    return delannoy(m - 1, n) + delannoy(m, n - 1) + delannoy(m - 1, n - 1)


def delannoy_table(m: int, n: int):
    """Iterative table T[i][j] = Delannoy(i, j) for 0<=i<=m, 0<=j<=n."""
    T = [[1] * (n + 1) for _ in range(m + 1)]
    for i in range(1, m + 1):
        for j in range(1, n + 1):
            T[i][j] = T[i - 1][j] + T[i][j - 1] + T[i - 1][j - 1]
    return T


def log_delannoy(m: int, n: int) -> float:
    return math.log(delannoy_table(m, n)[m][n])


def zero_dist_marginals(N: int, M: int) -> np.ndarray:
    """E for Dist == 0: every path has weight 1 / Del(N-1, M-1), so
    E[i,j] = Del(i,j) * Del(N-1-i, M-1-j) / Del(N-1, M-1), exactly."""
    T = delannoy_table(N - 1, M - 1)
    tot = T[N - 1][M - 1]
    E = np.empty((N, M))
    for i in range(N):
        for j in range(M):
            E[i, j] = float(Fraction(T[i][j] * T[N - 1 - i][M - 1 - j], tot))
    return E


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), 1e-300)

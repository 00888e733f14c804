"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no Soft-DTW arithmetic: it only draws the input sequences,
so the oracle and the HIP path see bit-identical fp32 data.

* ``pair_batch``: x[B,N,D] then y[B,M,D], i.i.d. N(0,1) fp32, drawn from one
  CPU ``torch.Generator`` seeded with ``seed`` (the README "SoftDTW-CUDA
  (PyTorch + Numba)", section "Usage", draws its inputs with ``torch.randn``).
* ``block_waves``: K random-phase square waves of length T with D channels,
  amplitude +-1 plus N(0, noise^2) noise (review page "SoftDTW-CUDA-Torch",
  Figure 2: a barycenter of synthetic block-wave data).  Reading: period 50,
  phase uniform on {0..period-1} per (sequence, channel), noise std 0.1.
"""
from __future__ import annotations

import torch


def pair_batch(B: int, N: int, M: int, D: int, seed: int = 0):
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn((B, N, D), dtype=torch.float32, generator=g)
    y = torch.randn((B, M, D), dtype=torch.float32, generator=g)
    return x, y


def block_waves(K: int = 10, T: int = 100, D: int = 3, seed: int = 0,
                period: int = 50, noise: float = 0.1):
    g = torch.Generator().manual_seed(int(seed))
    phase = torch.randint(0, period, (K, 1, D), generator=g)
    t = torch.arange(T).view(1, T, 1)
    sq = torch.where(((t + phase) % period) < (period // 2), 1.0, -1.0)
    eps = torch.randn((K, T, D), dtype=torch.float32, generator=g) * noise
    return (sq.to(torch.float32) + eps).contiguous()

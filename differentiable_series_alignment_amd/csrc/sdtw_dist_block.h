// Squared Euclidean distance block on fp64 MFMA (gfx950), shared by the
// distance kernel and the distance workers of the small-grid sweep kernel.
// See sdtw_dist.hip for the method; here only the block routine.
#pragma once
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

constexpr int kDT = 128;                 // output block edge per workgroup
constexpr int kDKC = 16;                 // features per slab
constexpr int kDPK = kDKC + 4;           // slab row pitch (floats)
constexpr int kDTP = kDT + 16;           // output block row pitch (floats)
constexpr int kDSlab = 2 * kDT * kDPK;   // x and y rows of one slab (floats)
constexpr int kDLds = (2 * kDSlab > kDT * kDTP ? 2 * kDSlab : kDT * kDTP);

// One 128 x 128 block (rows bi0.., columns bj0..) of pair b.  Threads 0..255
// of the workgroup compute; any further threads only take part in the
// barriers.  SKEW: band-step output (else row-major [B,N,M]); COH: the
// stores are device-coherent (they bypass the per-XCD caches, for readers
// in the same launch).  smem: kDLds floats.
template <bool SKEW, bool COH>
__device__ __forceinline__ void dist_block(const float* __restrict__ x,
                                           const float* __restrict__ y,
                                           float* __restrict__ dist, int64_t b, int64_t bi0,
                                           int64_t bj0, int64_t N, int64_t M, int64_t D,
                                           int64_t S, int nbands, float* smem) {
  const bool act = threadIdx.x < 256;
  // Two slab buffers, each [kDT][kDPK] x rows then [kDT][kDPK] y rows; the
  // finished block [kDT][kDTP] overlays them at the end.
  float* const tile = smem;
  const int l = lane_id();
  const int w = threadIdx.x >> 6;
  const int wr = w >> 1, wc = w & 1;      // this wave's 64x64 quarter
  const int r = l & 15, kk = l >> 4;
  const float* xb = x + b * N * D;
  const float* yb = y + b * M * D;

  // Staging: thread t moves elements t + 256q (q < 8) of each 128 x 16
  // slab; rows outside the grid and features >= D are stored as zeros.
  constexpr int kQ = kDT * kDKC / 256;
  float sx[kQ], sy[kQ];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      const int row = e / kDKC, col = e % kDKC;
      const int64_t d = k0 + col;
      const int64_t gi = bi0 + row, gj = bj0 + row;
      const bool dok = d < D;
      const float vx = xb[(gi < N ? gi : 0) * D + (dok ? d : 0)];
      const float vy = yb[(gj < M ? gj : 0) * D + (dok ? d : 0)];
      sx[q] = (dok && gi < N) ? vx : 0.f;
      sy[q] = (dok && gj < M) ? vy : 0.f;
    }
  };
  auto stash = [&](int buf) {
    float* xs = smem + buf * kDSlab;
    float* ys = xs + kDT * kDPK;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      xs[(e / kDKC) * kDPK + e % kDKC] = sx[q];
      ys[(e / kDKC) * kDPK + e % kDKC] = sy[q];
    }
  };

  v4d acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4d){0.0, 0.0, 0.0, 0.0};
  double nx[4] = {0, 0, 0, 0}, ny[4] = {0, 0, 0, 0};
  const int64_t steps = (D + 3) / 4;
  // Double-buffered slabs: slab k is read from buffer k & 1 while slab k+1
  // is written into the other one, and slab k+2 is fetched into registers;
  // one barrier per slab.
  const int nslab = (int)((D + kDKC - 1) / kDKC);
  if (act) {
    fetch(0);
    stash(0);
    if (nslab > 1) fetch(kDKC);
  }
  __syncthreads();
  for (int k = 0; k < nslab; ++k) {
    if (act) {
    const float* xa = smem + (k & 1) * kDSlab + (wr * 64 + r) * kDPK + kk;
    const float* yb_l = smem + (k & 1) * kDSlab + kDT * kDPK + (wc * 64 + r) * kDPK + kk;
    const int64_t s0 = (int64_t)k * (kDKC / 4);
    const int ns = (int)(steps - s0 < kDKC / 4 ? steps - s0 : kDKC / 4);
    for (int sl = 0; sl < ns; ++sl) {  // step s = s0 + sl, feature d = 4s + kk
      double a[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = (double)xa[16 * i * kDPK + 4 * sl];
        bv[i] = (double)yb_l[16 * i * kDPK + 4 * sl];
        nx[i] = fma(a[i], a[i], nx[i]);
        ny[i] = fma(bv[i], bv[i], ny[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (k + 1 < nslab) stash((k + 1) & 1);
    if (k + 2 < nslab) fetch((int64_t)(k + 2) * kDKC);
    }
    __syncthreads();
  }
  if (act) {
  // Complete the norms over the four k lane groups (lanes r, r+16, r+32, r+48).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nx[i] += __shfl_xor(nx[i], 16, 64);
    nx[i] += __shfl_xor(nx[i], 32, 64);
    ny[i] += __shfl_xor(ny[i], 16, 64);
    ny[i] += __shfl_xor(ny[i], 32, 64);
  }
  // Dist = max(0, |x|^2 + |y|^2 - 2 x.y), rounded once to fp32, into the
  // LDS block (which now overlays the slabs; the loop ended on a barrier).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = 4 * e + kk;
      const double nxr = __shfl(nx[i], rl, 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        double v = nxr + ny[j] - 2.0 * acc[i][j][e];
        v = v > 0.0 ? v : 0.0;
        tile[(wr * 64 + 16 * i + rl) * kDTP + wc * 64 + 16 * j + r] = (float)v;
      }
    }
  }
  __syncthreads();
  if (!act) return;
  if (SKEW) {
    // Band bb of the block (64 rows, columns bj0 .. bj0+127) covers steps
    // bj0 + p, p = 0..190, of that band; lane l of step p holds column
    // bj0 + p - l.  Per pass, thread t moves lanes l0..l0+3 (l0 = 4(t%16))
    // of step p = 16*pass + t/16: one 16-byte store when all four cells lie
    // in the block, single words at its diagonal edges.  A wave writes four
    // whole steps (1 KiB) per pass; the LDS reads of a pass do not wait on
    // the stores of the previous one.
    const int t = (int)threadIdx.x;
    const int l0 = 4 * (t & 15);
    const int cmax = (int)(M - bj0 < kDT ? M - bj0 : kDT);   // block columns in the grid
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int64_t band = (bi0 >> 6) + bb;
      if (band >= nbands) break;
      float* bandp = dist + ((b * nbands + band) * S + bj0 + kSkewOff) * 64 + l0;
      const float* tb = tile + (64 * bb + l0) * kDTP;
#pragma unroll 4
      for (int pass = 0; pass < (kDT + 63 + 15) / 16; ++pass) {
        const int p = 16 * pass + (t >> 4);
        float v[4];
        bool ok[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cl = p - l0 - j;
          ok[j] = cl >= 0 && cl < cmax;
          v[j] = tb[j * kDTP + (ok[j] ? cl : 0)];
        }
        float* dst = bandp + (int64_t)p * 64;
        if (COH) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ok[j])
              __hip_atomic_store(dst + j, v[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (ok[0] && ok[3]) {   // the valid lanes of a step are contiguous
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ok[j]) dst[j] = v[j];
        }
      }
    }
  } else {
    float* ob = dist + b * N * M;
    for (int rr = w; rr < kDT; rr += 4) {
      const int64_t gi = bi0 + rr;
      if (gi >= N) break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t gj = bj0 + l + 64 * h;
        if (gj < M) ob[gi * M + gj] = tile[rr * kDTP + l + 64 * h];
      }
    }
  }
}

}  // namespace sdtw

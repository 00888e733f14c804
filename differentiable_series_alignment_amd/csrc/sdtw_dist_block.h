// Squared Euclidean distance block on fp64 MFMA (gfx950): the routine the
// distance kernels run per block.  See sdtw_dist.hip for the method.
#pragma once
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

constexpr int kDT = 128;                 // output block width (columns)
constexpr int kDTP = kDT + 16;           // output block row pitch (floats)

// Staging of the operands.  KC = 16: slabs of 16 features, double-buffered,
// any D.  KC = 64 (D a multiple of 4, at most 64): all features at once,
// single-buffered, loaded as 16-byte vectors; one barrier before the
// matrix loop instead of one per slab.
template <int KC>
struct DistStage {
  static constexpr int kPK = KC + 4;     // row pitch (floats)
  static constexpr int kBufs = KC == 16 ? 2 : 1;
};

// LDS floats of a block of TR rows (64 or 128) x kDT columns: the slab
// buffers of TR x rows and kDT y rows each, which the finished block
// [TR][kDTP] overlays at the end.
template <int TR, int KC = 16>
struct DistTile {
  static constexpr int kSlab = (TR + kDT) * DistStage<KC>::kPK;
  static constexpr int kLds = (DistStage<KC>::kBufs * kSlab > TR * kDTP
                                   ? DistStage<KC>::kBufs * kSlab : TR * kDTP);
};

// One TR x 128 block (rows bi0.., columns bj0..) of pair b, computed by a
// 256-thread workgroup.  The four waves split the block into TR/64 x 4/(TR/64)
// parts of 64 rows each (64 x 64 for TR = 128, 64 x 32 for TR = 64).
// SKEW: band-step output (else row-major [B,N,M]).  smem: DistTile<TR>::kLds
// floats.
template <int TR, bool SKEW, int KC = 16>
__device__ __forceinline__ void dist_block(const float* __restrict__ x,
                                           const float* __restrict__ y,
                                           float* __restrict__ dist, int64_t b, int64_t bi0,
                                           int64_t bj0, int64_t N, int64_t M, int64_t D,
                                           int64_t S, int nbands, float* smem) {
  static_assert(TR == 64 || TR == 128, "block height");
  static_assert(KC == 16 || KC == 64, "features per slab");
  constexpr int kDKC = KC;
  constexpr int kDPK = DistStage<KC>::kPK;
  constexpr int WR = TR / 64;            // wave rows
  constexpr int WC = 4 / WR;             // wave columns
  constexpr int CW = kDT / WC;           // columns per wave
  constexpr int NJ = CW / 16;            // 16-column tiles per wave
  constexpr int kSlab = DistTile<TR, KC>::kSlab;
  float* const tile = smem;
  const int l = lane_id();
  const int w = threadIdx.x >> 6;
  const int wr = w / WC, wc = w % WC;    // this wave's part
  const int r = l & 15, kk = l >> 4;
  const float* xb = x + b * N * D;
  const float* yb = y + b * M * D;

  // Staging (KC = 16): thread t moves elements t + 256q of the TR x 16 x
  // slab and of the 128 x 16 y slab; rows outside the grid and features >= D
  // are stored as zeros.  (KC = 64: see stage_all below.)
  constexpr int kQX = KC == 16 ? TR * kDKC / 256 : 1, kQY = KC == 16 ? kDT * kDKC / 256 : 1;
  float sx[kQX], sy[kQY];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < kQY; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      const int row = e / kDKC, col = e % kDKC;
      const int64_t d = k0 + col;
      const bool dok = d < D;
      if (q < kQX) {
        const int64_t gi = bi0 + row;
        const float vx = xb[(gi < N ? gi : 0) * D + (dok ? d : 0)];
        sx[q < kQX ? q : 0] = (dok && gi < N) ? vx : 0.f;
      }
      const int64_t gj = bj0 + row;
      const float vy = yb[(gj < M ? gj : 0) * D + (dok ? d : 0)];
      sy[q] = (dok && gj < M) ? vy : 0.f;
    }
  };
  auto stash = [&](int buf) {
    float* xs = smem + buf * kSlab;
    float* ys = xs + TR * kDPK;
#pragma unroll
    for (int q = 0; q < kQY; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      if (q < kQX) xs[(e / kDKC) * kDPK + e % kDKC] = sx[q < kQX ? q : 0];
      ys[(e / kDKC) * kDPK + e % kDKC] = sy[q];
    }
  };

  v4d acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (v4d){0.0, 0.0, 0.0, 0.0};
  double nx[4] = {0, 0, 0, 0}, ny[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) ny[j] = 0.0;
  const int64_t steps = (D + 3) / 4;
  // KC = 64: chunks of 64 features (D a multiple of 4), single-buffered:
  // thread t moves 16-byte vectors t + 256q (row v / 16, features c0 + 4 (v %
  // 16) ..) of the block's TR x rows and 128 y rows, all loads issued before
  // any is stored; rows outside the grid and features >= D are stored as
  // zeros.  A later chunk is loaded once every wave is done with the
  // previous one (two barriers per chunk; other workgroups on the CU hide
  // the load; nothing is held in registers across the matrix loop).
  constexpr int kVX = KC == 64 ? TR * 16 / 256 : 1, kVY = KC == 64 ? kDT * 16 / 256 : 1;
  float4 vx[kVX], vy[kVY];
  auto load64 = [&](int64_t c0) {
#pragma unroll
    for (int q = 0; q < kVX; ++q) {
      const int v = (int)threadIdx.x + 256 * q;
      const int row = v >> 4;
      const int64_t d = c0 + 4 * (v & 15);
      const int64_t gi = bi0 + row;
      const bool ok = gi < N && d < D;
      const float4 t = *reinterpret_cast<const float4*>(xb + (ok ? gi * D + d : 0));
      vx[q] = ok ? t : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < kVY; ++q) {
      const int v = (int)threadIdx.x + 256 * q;
      const int row = v >> 4;
      const int64_t d = c0 + 4 * (v & 15);
      const int64_t gj = bj0 + row;
      const bool ok = gj < M && d < D;
      const float4 t = *reinterpret_cast<const float4*>(yb + (ok ? gj * D + d : 0));
      vy[q] = ok ? t : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store64 = [&]() {
    float* xs = smem;
    float* ys = xs + TR * kDPK;
#pragma unroll
    for (int q = 0; q < kVX; ++q) {
      const int v = (int)threadIdx.x + 256 * q;
      *reinterpret_cast<float4*>(xs + (v >> 4) * kDPK + 4 * (v & 15)) = vx[q];
    }
#pragma unroll
    for (int q = 0; q < kVY; ++q) {
      const int v = (int)threadIdx.x + 256 * q;
      *reinterpret_cast<float4*>(ys + (v >> 4) * kDPK + 4 * (v & 15)) = vy[q];
    }
  };
  const int nslab = (int)((D + kDKC - 1) / kDKC);
  if constexpr (KC == 64) {
    load64(0);
    store64();
  } else {
    // Double-buffered slabs: slab k is read from buffer k & 1 while slab k+1
    // is written into the other one, and slab k+2 is fetched into registers;
    // one barrier per slab.
    fetch(0);
    stash(0);
    if (nslab > 1) fetch(kDKC);
  }
  __syncthreads();
  for (int k = 0; k < nslab; ++k) {
    const int buf = KC == 16 ? (k & 1) : 0;
    const float* xa = smem + buf * kSlab + (wr * 64 + r) * kDPK + kk;
    const float* yb_l = smem + buf * kSlab + TR * kDPK + (wc * CW + r) * kDPK + kk;
    const int64_t s0 = (int64_t)k * (kDKC / 4);
    const int ns = (int)(steps - s0 < kDKC / 4 ? steps - s0 : kDKC / 4);
    for (int sl = 0; sl < ns; ++sl) {  // step s = s0 + sl, feature d = 4s + kk
      double a[4], bv[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = (double)xa[16 * i * kDPK + 4 * sl];
        nx[i] = fma(a[i], a[i], nx[i]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        bv[j] = (double)yb_l[16 * j * kDPK + 4 * sl];
        ny[j] = fma(bv[j], bv[j], ny[j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (KC == 16) {
      if (k + 1 < nslab) stash((k + 1) & 1);
      if (k + 2 < nslab) fetch((int64_t)(k + 2) * kDKC);
    } else {
      if (k + 1 < nslab) {
        __syncthreads();   // every wave is done with chunk k
        load64((int64_t)(k + 1) * kDKC);
        store64();
      }
    }
    __syncthreads();
  }
  // Complete the norms over the four k lane groups (lanes r, r+16, r+32, r+48).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nx[i] += __shfl_xor(nx[i], 16, 64);
    nx[i] += __shfl_xor(nx[i], 32, 64);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    ny[j] += __shfl_xor(ny[j], 16, 64);
    ny[j] += __shfl_xor(ny[j], 32, 64);
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
      for (int j = 0; j < NJ; ++j) {
        double v = nxr + ny[j] - 2.0 * acc[i][j][e];
        v = v > 0.0 ? v : 0.0;
        tile[(wr * 64 + 16 * i + rl) * kDTP + wc * CW + 16 * j + r] = (float)v;
      }
    }
  __syncthreads();
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
    for (int bb = 0; bb < WR; ++bb) {
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
        if (ok[0] && ok[3]) {   // the valid lanes of a step are contiguous
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
    for (int rr = w; rr < TR; rr += 4) {
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

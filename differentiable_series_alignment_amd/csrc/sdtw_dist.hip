// Squared Euclidean distance tile on fp64 MFMA (gfx950).
//
// Dist[b,i,j] = ||x_i - y_j||^2 = |x_i|^2 + |y_j|^2 - 2 x_i.y_j, the
// distance of the README "SoftDTW-CUDA (PyTorch + Numba)" ("Usage", unfused
// mode: an explicit distance tensor; "Notes": never negative, hence the clamp
// at zero).  The dot products and norms are accumulated in fp64 (products of
// fp32 inputs are exact in fp64) and the result is rounded once to fp32, so
// the stored value is the fp32 nearest to the exact distance except for
// inputs within ~1e-13 relative of a rounding midpoint.
//
// Work split: a 256-thread workgroup owns a 64x64 block of (i,j) for one
// pair; each wave owns a 32x32 quarter as 2x2 tiles of
// v_mfma_f64_16x16x4_f64.  Operand lanes: A[r][k] sits in lane r + 16k,
// B[k][c] in lane c + 16k; the accumulator's element (4*e + l/16, l%16) sits
// in lane l, register e (checked on the hardware).  The contraction index k of step s is d = 4s + k.
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

// Finish one 16x16 accumulator tile: Dist = max(0, |x|^2 + |y|^2 - 2 x.y)
// rounded once to fp32.  Plain output goes to out[row * ldo + col]; the
// band-step output is staged in the workgroup's LDS tile first.
template <bool SKEW>
__device__ __forceinline__ void dist_tile_store(float* out, int64_t ldo,
                                                int64_t i0, int64_t j0,
                                                int64_t N, int64_t M,
                                                const v4d& acc, double nx_l,
                                                double ny_l, float* tile,
                                                int ti, int tj) {
  const int l = lane_id();
  const int col = l & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * e + (l >> 4);
    const double nx_row = __shfl(nx_l, row, 64);
    double v = nx_row + ny_l - 2.0 * acc[e];
    v = v > 0.0 ? v : 0.0;
    if (SKEW) {
      tile[(ti + row) * 64 + tj + col] = (float)v;
    } else {
      const int64_t gi = i0 + row, gj = j0 + col;
      if (gi < N && gj < M) out[gi * ldo + gj] = (float)v;
    }
  }
}

template <bool SKEW>
__global__ __launch_bounds__(256) void k_dist(const float* __restrict__ x,
                                              const float* __restrict__ y,
                                              float* __restrict__ dist,
                                              int64_t N, int64_t M, int64_t D,
                                              int64_t S) {
  // The workgroup's 64 x rows and 64 y rows pass through LDS in slabs of
  // KC feature columns (coalesced loads; the next slab is fetched into
  // registers while the current one feeds the MFMAs).  Rows outside the
  // grid and columns >= D are stored as zeros.
  constexpr int KC = 64, PK = KC + 4;
  __shared__ float xs[64 * PK], ys[64 * PK];
  __shared__ float tile[SKEW ? 64 * 64 : 1];
  const int l = lane_id();
  const int w = threadIdx.x >> 6;
  const int64_t b = blockIdx.z;
  const int64_t bi0 = (int64_t)blockIdx.y * 64, bj0 = (int64_t)blockIdx.x * 64;
  const int64_t i0 = bi0 + (w >> 1) * 32;
  const int64_t j0 = bj0 + (w & 1) * 32;
  const float* xb = x + b * N * D;
  const float* yb = y + b * M * D;
  const int r = l & 15, kk = l >> 4;
  const int ra = (w >> 1) * 32 + r, rb = (w & 1) * 32 + r;  // slab rows of this lane

  // Staging: thread t moves elements t + 256 q (q < 16) of each 64 x KC slab.
  float sx[16], sy[16];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      const int row = e / KC, col = e % KC;
      const int64_t d = k0 + col;
      const int64_t gi = bi0 + row, gj = bj0 + row;
      const bool dok = d < D;
      const float vx = xb[(gi < N ? gi : 0) * D + (dok ? d : 0)];
      const float vy = yb[(gj < M ? gj : 0) * D + (dok ? d : 0)];
      sx[q] = (dok && gi < N) ? vx : 0.f;
      sy[q] = (dok && gj < M) ? vy : 0.f;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = (int)threadIdx.x + 256 * q;
      xs[(e / KC) * PK + e % KC] = sx[q];
      ys[(e / KC) * PK + e % KC] = sy[q];
    }
  };

  v4d acc00 = {0, 0, 0, 0}, acc01 = acc00, acc10 = acc00, acc11 = acc00;
  double nxa0 = 0, nxa1 = 0, nyb0 = 0, nyb1 = 0;
  const int64_t steps = (D + 3) / 4;
  fetch(0);
  for (int64_t k0 = 0; k0 < D; k0 += KC) {
    __syncthreads();
    stash();
    __syncthreads();
    if (k0 + KC < D) fetch(k0 + KC);
    const int64_t s0 = k0 / 4;
    const int ns = (int)(steps - s0 < KC / 4 ? steps - s0 : KC / 4);
    for (int sl = 0; sl < ns; ++sl) {  // step s = s0 + sl, feature d = 4s + kk
      const int c = 4 * sl + kk;
      const double a0 = (double)xs[ra * PK + c];
      const double a1 = (double)xs[(ra + 16) * PK + c];
      const double b0 = (double)ys[rb * PK + c];
      const double b1 = (double)ys[(rb + 16) * PK + c];
      nxa0 = fma(a0, a0, nxa0);
      nxa1 = fma(a1, a1, nxa1);
      nyb0 = fma(b0, b0, nyb0);
      nyb1 = fma(b1, b1, nyb1);
      acc00 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc11, 0, 0, 0);
    }
  }
  // Complete the norms over the four k lane groups (lanes r, r+16, r+32, r+48).
  nxa0 += __shfl_xor(nxa0, 16, 64);
  nxa0 += __shfl_xor(nxa0, 32, 64);
  nxa1 += __shfl_xor(nxa1, 16, 64);
  nxa1 += __shfl_xor(nxa1, 32, 64);
  nyb0 += __shfl_xor(nyb0, 16, 64);
  nyb0 += __shfl_xor(nyb0, 32, 64);
  nyb1 += __shfl_xor(nyb1, 16, 64);
  nyb1 += __shfl_xor(nyb1, 32, 64);

  float* ob = dist + (SKEW ? 0 : b * N * M);
  const int ti = (w >> 1) * 32, tj = (w & 1) * 32;
  dist_tile_store<SKEW>(ob, M, i0, j0, N, M, acc00, nxa0, nyb0, tile, ti, tj);
  dist_tile_store<SKEW>(ob, M, i0, j0 + 16, N, M, acc01, nxa0, nyb1, tile, ti, tj + 16);
  dist_tile_store<SKEW>(ob, M, i0 + 16, j0, N, M, acc10, nxa1, nyb0, tile, ti + 16, tj);
  dist_tile_store<SKEW>(ob, M, i0 + 16, j0 + 16, N, M, acc11, nxa1, nyb1, tile, ti + 16, tj + 16);
  if (SKEW) {
    // The 64x64 block (one band, columns c0..c0+63) covers steps
    // c0+p, p = 0..126, of the band; lane l of step p holds column
    // c0 + p - l.  Each store writes one step's contiguous lane run.
    __syncthreads();
    const int64_t band = blockIdx.y, c0 = (int64_t)blockIdx.x * 64;
    const int64_t nb = gridDim.y;
    float* bandp = dist + ((b * nb + band) * S + c0 + kSkewOff) * 64;
    for (int p = w; p < 127; p += 4) {
      const int cl = p - l;
      if (cl >= 0 && cl < 64 && c0 + cl < M) bandp[(int64_t)p * 64 + l] = tile[l * 64 + cl];
    }
  }
}

hipError_t launch_dist(const float* x, const float* y, float* dist, int64_t B,
                       int64_t N, int64_t M, int64_t D, hipStream_t stream) {
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)B);
  hipLaunchKernelGGL(k_dist<false>, grid, dim3(256), 0, stream, x, y, dist, N, M, D,
                     (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_dist_skew(const float* x, const float* y, float* dsk, int64_t B,
                            int64_t N, int64_t M, int64_t D, int64_t S,
                            hipStream_t stream) {
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)B);
  hipLaunchKernelGGL(k_dist<true>, grid, dim3(256), 0, stream, x, y, dsk, N, M, D, S);
  return hipGetLastError();
}

// Band-step E -> plain [B,N,M] (the optional alignment-matrix output).
__global__ __launch_bounds__(256) void k_unskew(const float* __restrict__ esk,
                                                float* __restrict__ out, int64_t N,
                                                int64_t M, int64_t S, int nbands) {
  const int64_t b = blockIdx.z;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= M) return;
  for (int64_t r = blockIdx.y; r < N; r += gridDim.y)
    out[(b * N + r) * M + c] = esk[skew_index(b, r, c, nbands, S)];
}

hipError_t launch_unskew(const float* esk, float* out, int64_t B, int64_t N,
                         int64_t M, int64_t S, hipStream_t s) {
  dim3 grid((unsigned)((M + 255) / 256), (unsigned)(N < 4096 ? N : 4096), (unsigned)B);
  hipLaunchKernelGGL(k_unskew, grid, dim3(256), 0, s, esk, out, N, M, S,
                     (int)((N + 63) / 64));
  return hipGetLastError();
}

}  // namespace sdtw

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
// B[k][c] in lane c + 16k; the accumulator's element (4*(l/16)+e, l%16) sits
// in lane l, register e.  The contraction index k of step s is d = 4s + k.
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

__device__ __forceinline__ void dist_tile_store(float* out, int64_t ldo,
                                                int64_t i0, int64_t j0,
                                                int64_t N, int64_t M,
                                                const v4d& acc, double nx_l,
                                                double ny_l) {
  const int l = lane_id();
  const int col = l & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * (l >> 4) + e;
    const double nx_row = __shfl(nx_l, row, 64);
    double v = nx_row + ny_l - 2.0 * acc[e];
    v = v > 0.0 ? v : 0.0;
    const int64_t gi = i0 + row, gj = j0 + col;
    if (gi < N && gj < M) out[gi * ldo + gj] = (float)v;
  }
}

__global__ __launch_bounds__(256) void k_dist(const float* __restrict__ x,
                                              const float* __restrict__ y,
                                              float* __restrict__ dist,
                                              int64_t N, int64_t M, int64_t D) {
  const int l = lane_id();
  const int w = threadIdx.x >> 6;
  const int64_t b = blockIdx.z;
  const int64_t i0 = (int64_t)blockIdx.y * 64 + (w >> 1) * 32;
  const int64_t j0 = (int64_t)blockIdx.x * 64 + (w & 1) * 32;
  const float* xb = x + b * N * D;
  const float* yb = y + b * M * D;
  const int r = l & 15, kk = l >> 4;

  // Rows / columns this lane feeds into the A and B operands.
  const int64_t ia0 = i0 + r, ia1 = i0 + 16 + r;
  const int64_t jb0 = j0 + r, jb1 = j0 + 16 + r;
  const bool va0 = ia0 < N, va1 = ia1 < N, vb0 = jb0 < M, vb1 = jb1 < M;
  const float* pa0 = xb + (va0 ? ia0 : 0) * D;
  const float* pa1 = xb + (va1 ? ia1 : 0) * D;
  const float* pb0 = yb + (vb0 ? jb0 : 0) * D;
  const float* pb1 = yb + (vb1 ? jb1 : 0) * D;

  v4d acc00 = {0, 0, 0, 0}, acc01 = acc00, acc10 = acc00, acc11 = acc00;
  double nxa0 = 0, nxa1 = 0, nyb0 = 0, nyb1 = 0;
  const int64_t steps = (D + 3) / 4;
#pragma unroll 4
  for (int64_t s = 0; s < steps; ++s) {
    const int64_t d = 4 * s + kk;
    const bool vd = d < D;
    const double a0 = (vd && va0) ? (double)pa0[d] : 0.0;
    const double a1 = (vd && va1) ? (double)pa1[d] : 0.0;
    const double b0 = (vd && vb0) ? (double)pb0[d] : 0.0;
    const double b1 = (vd && vb1) ? (double)pb1[d] : 0.0;
    nxa0 = fma(a0, a0, nxa0);
    nxa1 = fma(a1, a1, nxa1);
    nyb0 = fma(b0, b0, nyb0);
    nyb1 = fma(b1, b1, nyb1);
    acc00 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc00, 0, 0, 0);
    acc01 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc01, 0, 0, 0);
    acc10 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc10, 0, 0, 0);
    acc11 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc11, 0, 0, 0);
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

  float* ob = dist + b * N * M;
  dist_tile_store(ob, M, i0, j0, N, M, acc00, nxa0, nyb0);
  dist_tile_store(ob, M, i0, j0 + 16, N, M, acc01, nxa0, nyb1);
  dist_tile_store(ob, M, i0 + 16, j0, N, M, acc10, nxa1, nyb0);
  dist_tile_store(ob, M, i0 + 16, j0 + 16, N, M, acc11, nxa1, nyb1);
}

hipError_t launch_dist(const float* x, const float* y, float* dist, int64_t B,
                       int64_t N, int64_t M, int64_t D, hipStream_t stream) {
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)B);
  hipLaunchKernelGGL(k_dist, grid, dim3(256), 0, stream, x, y, dist, N, M, D);
  return hipGetLastError();
}

}  // namespace sdtw

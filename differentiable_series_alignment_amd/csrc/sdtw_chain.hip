// Chain rule of Soft-DTW through the squared Euclidean distance (gfx950).
//
// With E = dloss/dDist (the alignment matrix) and Dist = ||x_i - y_j||^2:
//   dx[b,i,:] = 2 gl[b] (rowsum_i(E) x_i - sum_j E[i,j] y_j),
//   dy[b,j,:] = 2 gl[b] (colsum_j(E) y_j - sum_i E[i,j] x_i),
// i.e. two batched contractions E.Y and E^T.X (README "SoftDTW-CUDA (PyTorch +
// Numba)", "Usage": gradients of loss_fn(x, y).mean() reach x and y).
//
// One wave owns 32 output rows and all of D (up to 256 columns per pass, as
// 32x32 tiles of v_mfma_f32_32x32x2_f32 accumulated over the contraction
// index K in steps of 2).  Operand lanes: A[r][k] in lane r + 32k, B[k][c] in
// lane c + 32k; accumulator element (8*(e/4) + 4*(l/32) + e%4, l%32) in lane
// l, register e.  Step s contracts k = s (lanes 0..31) and k = s + Kh (lanes
// 32..63), Kh = ceil(K/2), so each lane walks one contiguous half of K.
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

// ROLE 0: rows i, out = dx, own = x, other = y, A[r][k] = E[i0+r][k].
// ROLE 1: rows j, out = dy, own = y, other = x, A[r][k] = E[k][j0+r].
template <int ROLE, int NT>
__device__ __forceinline__ void chain_wave(const float* __restrict__ Eb,
                                           const float* __restrict__ own,
                                           const float* __restrict__ other,
                                           float* __restrict__ out, float g2,
                                           int64_t rows, int64_t K, int64_t D,
                                           int64_t ldE, int64_t r0, int64_t d0) {
  const int l = lane_id();
  const int rl = l & 31, hk = l >> 5;
  const int64_t Kh = (K + 1) / 2;
  const int64_t row = r0 + rl;
  const bool row_ok = row < rows;
  v16f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  float rsum = 0.f;
  int64_t dcol[NT];
  bool dok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    dcol[t] = d0 + 32 * t + rl;
    dok[t] = dcol[t] < D;
  }
  for (int64_t s = 0; s < Kh; ++s) {
    const int64_t k = s + hk * Kh;
    const bool kok = k < K;
    float av = 0.f;
    if (kok && row_ok) av = (ROLE == 0) ? Eb[row * ldE + k] : Eb[k * ldE + row];
    rsum += av;
    const float* orow = other + (kok ? k : 0) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float bv = (kok && dok[t]) ? orow[dcol[t]] : 0.f;
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[t], 0, 0, 0);
    }
  }
  rsum += __shfl_xor(rsum, 32, 64);
  // Row sums of the accumulator rows this lane holds (all lanes shuffle).
  float rs[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) rs[e] = __shfl(rsum, 8 * (e >> 2) + 4 * hk + (e & 3), 64);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t orw = r0 + 8 * (e >> 2) + 4 * hk + (e & 3);
      if (dok[t] && orw < rows) {
        const float ov = own[orw * D + dcol[t]];
        out[orw * D + dcol[t]] = g2 * (rs[e] * ov - acc[t][e]);
      }
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256) void k_chain(const float* __restrict__ E,
                                               const float* __restrict__ x,
                                               const float* __restrict__ y,
                                               const float* __restrict__ gl,
                                               float* __restrict__ gx,
                                               float* __restrict__ gy,
                                               int64_t N, int64_t M, int64_t D,
                                               int xblocks, int64_t d0) {
  const int w = threadIdx.x >> 6;
  const int64_t b = blockIdx.y;
  const float g2 = 2.f * gl[b];
  const float* Eb = E + b * N * M;
  if ((int)blockIdx.x < xblocks) {
    if (!gx) return;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + w) * 32;
    if (r0 >= N) return;
    chain_wave<0, NT>(Eb, x + b * N * D, y + b * M * D, gx + b * N * D, g2, N,
                      M, D, M, r0, d0);
  } else {
    if (!gy) return;
    const int64_t r0 = ((int64_t)(blockIdx.x - xblocks) * 4 + w) * 32;
    if (r0 >= M) return;
    chain_wave<1, NT>(Eb, y + b * M * D, x + b * N * D, gy + b * M * D, g2, M,
                      N, D, M, r0, d0);
  }
}

hipError_t launch_chain(const float* E, const float* x, const float* y,
                        const float* gl, float* gx, float* gy, int64_t B,
                        int64_t N, int64_t M, int64_t D, hipStream_t s) {
  const int xblocks = (int)((N + 127) / 128);
  const int yblocks = (int)((M + 127) / 128);
  dim3 grid((unsigned)(xblocks + yblocks), (unsigned)B);
  for (int64_t d0 = 0; d0 < D; d0 += 256) {
    const int64_t dw = D - d0 < 256 ? D - d0 : 256;
    const int nt = (int)((dw + 31) / 32);
    if (nt <= 1)
      hipLaunchKernelGGL(k_chain<1>, grid, dim3(256), 0, s, E, x, y, gl, gx, gy, N, M, D, xblocks, d0);
    else if (nt <= 2)
      hipLaunchKernelGGL(k_chain<2>, grid, dim3(256), 0, s, E, x, y, gl, gx, gy, N, M, D, xblocks, d0);
    else if (nt <= 4)
      hipLaunchKernelGGL(k_chain<4>, grid, dim3(256), 0, s, E, x, y, gl, gx, gy, N, M, D, xblocks, d0);
    else
      hipLaunchKernelGGL(k_chain<8>, grid, dim3(256), 0, s, E, x, y, gl, gx, gy, N, M, D, xblocks, d0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sdtw

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
// Work split: a 256-thread workgroup owns a 128x128 block of (i,j) for one
// pair, each wave a 64x64 quarter as 4x4 tiles of v_mfma_f64_16x16x4_f64
// (16 independent accumulation chains); or a 64x128 block, each wave a
// 64x32 part as 4x2 tiles (the band-step kernel's choice depends on the
// grid size, see dist_rows).  Operand
// lanes: A[r][k] sits in lane r + 16k, B[k][c] in lane c + 16k; the
// accumulator's element (4*e + l/16, l%16) sits in lane l, register e
// (checked on the hardware).  The contraction index k of step s is
// d = 4s + k.  The x and y rows pass through LDS: where D is a multiple of
// 4 (and the rows are 16-byte aligned) in chunks of 64 features moved as
// 16-byte vectors, every load of a chunk issued before any is stored and one
// barrier before the matrix loop; otherwise in double-buffered slabs of 16
// features (the next slab fetched into registers while the current one feeds
// the MFMAs).  The finished block is staged in LDS (over the operands) and
// leaves either row-major or in the band-step layout of the dynamic
// programme.
#include "sdtw_dist_block.h"

namespace sdtw {

template <int TR, bool SKEW, int KC>
__global__ __launch_bounds__(256, 2) void k_dist(const float* __restrict__ x,
                                              const float* __restrict__ y,
                                              float* __restrict__ dist,
                                              int64_t N, int64_t M, int64_t D,
                                              int64_t S, int nbands,
                                              unsigned* __restrict__ zero, int64_t nzero,
                                              uint64_t* __restrict__ empty, int64_t nempty) {
  __shared__ __align__(16) float smem[DistTile<TR, KC>::kLds];
  // Words the next kernels of the step expect to find cleared (their
  // control words and hand-off rows; a fresh workspace holds garbage),
  // spread over the grid.
  {
    const int64_t wg = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t stride = (int64_t)gridDim.x * gridDim.y * gridDim.z * 256;
    for (int64_t k = wg * 256 + threadIdx.x; k < nzero; k += stride) zero[k] = 0u;
    for (int64_t k = wg * 256 + threadIdx.x; k < nempty; k += stride) empty[k] = kHEmpty;
  }
  dist_block<TR, SKEW, KC>(x, y, dist, blockIdx.z, (int64_t)blockIdx.y * TR,
                       (int64_t)blockIdx.x * kDT, N, M, D, S, nbands, smem);
}

// Block height of the band-step distance kernel.  128-row blocks (two
// workgroups per CU, each wave 64 x 64) once they are more than the GPU has
// CUs (B=32, N=M=512: one round, 42.5 -> 34 us with the 64-feature chunks;
// 32 x 2048^2 and 32 x 4096 x 1000, D=128: 799 -> 765 and 781 -> 757 us);
// otherwise 64-row blocks, twice the workgroups, so that small batches
// still spread over every CU (32 x 256^2, D=256: 35.6 against 50.0 us).
static int dist_rows(int64_t B, int64_t N, int64_t M) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int64_t blocks128 = B * ((N + 127) / 128) * ((M + kDT - 1) / kDT);
  return blocks128 > cus ? 128 : 64;
}

// 64-feature chunks of 16-byte vectors (KC = 64) where rows are whole,
// aligned vectors.
static bool stage_all(const float* x, const float* y, int64_t D) {
  return D % 4 == 0 &&
         ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
}

hipError_t launch_dist(const float* x, const float* y, float* dist, int64_t B,
                       int64_t N, int64_t M, int64_t D, hipStream_t stream) {
  dim3 grid((unsigned)((M + kDT - 1) / kDT), (unsigned)((N + kDT - 1) / kDT), (unsigned)B);
  {
    TimedLaunch timed_("dist", stream);
    if (stage_all(x, y, D))
      hipLaunchKernelGGL((k_dist<128, false, 64>), grid, dim3(256), 0, stream, x, y, dist, N,
                         M, D, (int64_t)0, 0, (unsigned*)nullptr, (int64_t)0,
                         (uint64_t*)nullptr, (int64_t)0);
    else
      hipLaunchKernelGGL((k_dist<128, false, 16>), grid, dim3(256), 0, stream, x, y, dist, N,
                         M, D, (int64_t)0, 0, (unsigned*)nullptr, (int64_t)0,
                         (uint64_t*)nullptr, (int64_t)0);
  }
  return hipGetLastError();
}

hipError_t launch_dist_skew(const float* x, const float* y, float* dsk, int64_t B,
                            int64_t N, int64_t M, int64_t D, int64_t S, unsigned* zero,
                            int64_t nzero, double* empty, int64_t nempty, hipStream_t stream) {
  uint64_t* const eb = reinterpret_cast<uint64_t*>(empty);
  const int tr = dist_rows(B, N, M);
  dim3 grid((unsigned)((M + kDT - 1) / kDT), (unsigned)((N + tr - 1) / tr), (unsigned)B);
  {
    TimedLaunch timed_("dist_skew", stream);
    const int nb = (int)((N + 63) / 64);
    if (tr == 64 && stage_all(x, y, D))
      hipLaunchKernelGGL((k_dist<64, true, 64>), grid, dim3(256), 0, stream, x, y, dsk, N, M, D,
                         S, nb, zero, nzero, eb, nempty);
    else if (tr == 64)
      hipLaunchKernelGGL((k_dist<64, true, 16>), grid, dim3(256), 0, stream, x, y, dsk, N, M, D,
                         S, nb, zero, nzero, eb, nempty);
    else if (stage_all(x, y, D))
      hipLaunchKernelGGL((k_dist<128, true, 64>), grid, dim3(256), 0, stream, x, y, dsk, N, M,
                         D, S, nb, zero, nzero, eb, nempty);
    else
      hipLaunchKernelGGL((k_dist<128, true, 16>), grid, dim3(256), 0, stream, x, y, dsk, N, M,
                         D, S, nb, zero, nzero, eb, nempty);
  }
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
  {
    TimedLaunch timed_("unskew", s);
    hipLaunchKernelGGL(k_unskew, grid, dim3(256), 0, s, esk, out, N, M, S,
                       (int)((N + 63) / 64));
  }
  return hipGetLastError();
}

}  // namespace sdtw

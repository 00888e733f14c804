// Launch wrappers of the gfx950 Soft-DTW kernels (host side, internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdtw {

// Arguments of the wavefront dynamic-programme kernels.  Index spaces: the
// forward sweep walks the grid from (0,0) to (N-1,M-1); the reverse sweep
// walks it from (N-1,M-1) back to (0,0), i.e. the forward recurrence on both
// sequences reversed.  "Rows" and "columns" below are in the sweep's own
// space; arrays in memory are always in the original orientation.
struct DPArgs {
  const float* dist;    // [B,N,M] fp32 distances (unfused) or nullptr
  const float* x;       // [B,N,D] (fused)
  const float* y;       // [B,M,D] (fused)
  double* R;            // [B,N,M] fp64 forward state
  float* E;             // reverse: [B,N,M] alignment output (may alias dist)
  double* H;            // [B,nseg,M] fp64 bottom rows handed between segments
  unsigned* ctrl;       // [0] ticket; [1 + b*nseg + s] columns published by segment s
  double* loss64;       // [B] R[N,M] in fp64 (forward writes, reverse reads)
  float* loss;          // [B] (forward)
  const float* gl;      // [B] upstream gradients (fused reverse)
  float* gx;            // [B,N,D] (fused reverse)
  float* gy;            // [B,M,D] (fused reverse, accumulated atomically)
  int64_t N, M, D;
  int B, nbands, nseg;
  double k2;            // log2(e) / gamma
  double g_ln2;         // gamma * ln(2)
};

// Bands (64 rows each) per workgroup of the DP kernels.
constexpr int kBandsPerWG = 4;

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_dist(const float* x, const float* y, float* dist, int64_t B,
                       int64_t N, int64_t M, int64_t D, hipStream_t stream);
hipError_t launch_dp(const DPArgs& a, bool reverse, bool fused, hipStream_t s);
hipError_t launch_chain(const float* E, const float* x, const float* y,
                        const float* gl, float* gx, float* gy, int64_t B,
                        int64_t N, int64_t M, int64_t D, hipStream_t s);

}  // namespace sdtw

// Anti-diagonal wavefront kernels of the Soft-DTW dynamic programme (gfx950).
//
// Recurrence (Soft-DTW of Cuturi & Blondel, credited in the "Acknowledgments"
// of the README "SoftDTW-CUDA (PyTorch + Numba)"):
//   R[i,j] = Dist[i,j] + softmin_g(R[i-1,j-1], R[i-1,j], R[i,j-1]),
// with R[-1,-1] = 0 and every other out-of-grid cell +inf (0-based cells).
//
// The pages lift the 1024-length cap by running the anti-diagonals as tiles,
// one launch per anti-diagonal (review page "SoftDTW-CUDA-Torch", section
// "Proposed method"; README "Why This Implementation?").  Here a single launch
// runs the whole sweep for any N and M:
//  - one wave owns a band of 64 consecutive rows, lane l = row r0+l; at local
//    step t lane l computes column t-l, so the 64 cells of a step lie on one
//    anti-diagonal and each depends only on step t-1 and t-2 results;
//  - R[i-1,j] arrives from lane l-1 by a whole-wave DPP shift; lane 0 takes
//    it from the band above;
//  - the state of a cell is fp64; exp/log are the fp32 hardware ones applied
//    to fp64 differences (see softmin_cell);
//  - the kBandsPerWG bands of a workgroup advance in lock step, chunk by
//    chunk (CH steps), band w running LAG chunks behind band w-1 and reading
//    its top row from an LDS ring that band w-1's lane 63 fills;
//  - consecutive workgroups of one pair ("segments") hand the bottom row of
//    the segment over through global memory with agent-scope release/acquire
//    counters; workgroups take tickets in arrival order and a segment only
//    waits on a smaller ticket, so the wait always ends.
//
// The reverse sweep runs the same recurrence on both sequences reversed,
// which yields R'[i,j], the soft-DTW value of the suffix alignment from
// (i,j) to (N-1,M-1) that includes Dist[i,j].  In log space the alignment
// matrix is then
//   ln E[i,j] = (R[N-1,M-1] + Dist[i,j] - R[i,j] - R'[i,j]) / g,
// and E is exponentiated only at the end, cell by cell (the log-space
// backward with a final exp of the review page, section "Proposed method";
// the identity follows from splitting every alignment path at (i,j)).
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

constexpr int kCH = 16;                      // steps per chunk
constexpr int kLag = 2 + 62 / kCH;           // chunks between adjacent bands
constexpr int kRing = 128;                   // LDS ring columns per boundary
constexpr int kPub = 4;                      // chunks between global publishes
constexpr int kSlack = 64;                   // extra columns awaited at start
constexpr uint32_t kSpinCap = 1u << 25;      // polls before a wait gives up
static_assert(kRing >= (kLag + 3) * kCH, "LDS ring too small");

__global__ void k_zero_u32(unsigned* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void k_zero_f32(float* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <bool REV>
__global__ __launch_bounds__(kBandsPerWG * 64) void k_dp_unfused(DPArgs a) {
  constexpr int W = kBandsPerWG;
  __shared__ double ring[W > 1 ? W - 1 : 1][kRing];
  __shared__ unsigned s_ticket;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.ctrl[0], 1u);
  __syncthreads();
  const unsigned ticket = s_ticket;
  const int seg = (int)(ticket / (unsigned)a.B);
  const int b = (int)(ticket % (unsigned)a.B);

  const int64_t N = a.N, M = a.M;
  const int band = seg * W + w;
  const int nb_seg = min(W, a.nbands - seg * W);
  const bool active = w < nb_seg;
  const int64_t r0 = (int64_t)band * 64;
  const int64_t i = r0 + lane;                        // sweep-space row
  const bool row_ok = active && i < N;
  const int64_t orow = REV ? (N - 1 - (row_ok ? i : 0)) : (row_ok ? i : 0);
  const int qcount = (int)((M + 63 + kCH - 1) / kCH);
  const int qtot = qcount + kLag * (nb_seg - 1);
  const bool last_in_seg = (w == nb_seg - 1);
  const bool produce_global = active && last_in_seg && (seg + 1 < a.nseg);
  const bool consume_global = active && (w == 0) && (seg > 0);

  unsigned* prog_in = a.ctrl + 1 + (int64_t)b * a.nseg + (seg > 0 ? seg - 1 : 0);
  unsigned* prog_out = a.ctrl + 1 + (int64_t)b * a.nseg + seg;
  const double* Hin = a.H + ((int64_t)b * a.nseg + (seg > 0 ? seg - 1 : 0)) * M;
  double* Hout = a.H + ((int64_t)b * a.nseg + seg) * M;

  const int64_t rowoff = ((int64_t)b * N + orow) * M;
  const float* drow = a.dist + rowoff;
  double* Rrow = a.R + rowoff;
  float* Erow = REV ? a.E + rowoff : nullptr;
  const double k2 = a.k2, g_ln2 = a.g_ln2;
  const double rnm = REV ? a.loss64[b] : 0.0;

  double cur = kInf;
  double up = (lane == 0 && r0 == 0) ? 0.0 : kInf;  // diagonal input of step 0
  unsigned avail = 0;

  for (int Q = 0; Q < qtot; ++Q) {
    const int q = Q - kLag * w;
    if (active && q >= 0 && q < qcount) {
      const int64_t t0 = (int64_t)q * kCH;
      double top[kCH];
      if (r0 == 0) {
#pragma unroll
        for (int u = 0; u < kCH; ++u) top[u] = kInf;
      } else if (!consume_global) {
#pragma unroll
        for (int u = 0; u < kCH; ++u) top[u] = ring[w - 1][(t0 + u) & (kRing - 1)];
      } else {
        const unsigned need =
            (unsigned)imin64(M, t0 + kCH + (q == 0 ? kSlack : 0));
        if (avail < need) {
          // Bounded wait: the producer holds a smaller ticket and is running,
          // so it publishes within one segment's sweep; the cap only makes
          // sure every wave exits even if that ever failed (the result would
          // then be garbage, never a hang).
          unsigned v = 0;
          for (uint32_t spin = 0; spin < kSpinCap; ++spin) {
            v = __hip_atomic_load(prog_in, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if (v >= need) break;
            __builtin_amdgcn_s_sleep(2);
          }
          avail = v < need ? need : v;
        }
#pragma unroll
        for (int u = 0; u < kCH; ++u) {
          const int64_t col = t0 + u;
          top[u] = col < M ? Hin[col] : kInf;
        }
      }

      float dv[kCH];
      double rv[kCH];
#pragma unroll
      for (int u = 0; u < kCH; ++u) {
        const int64_t col = t0 + u - lane;
        const bool ok = row_ok && col >= 0 && col < M;
        const int64_t oc = REV ? (M - 1 - col) : col;
        dv[u] = ok ? drow[oc] : 0.f;
        if (REV) rv[u] = ok ? Rrow[oc] : 0.0;
      }

      double bottom[kCH];
#pragma unroll
      for (int u = 0; u < kCH; ++u) {
        const int64_t col = t0 + u - lane;
        const double upn = wave_shr1(cur, top[u]);
        const double diag = up;
        up = upn;
        double c = softmin_cell(diag, upn, cur, (double)dv[u], k2, g_ln2);
        c = col < 0 ? kInf : c;
        cur = c;
        bottom[u] = c;
        const bool ok = row_ok && col >= 0 && col < M;
        if (!REV) {
          if (ok) {
            Rrow[col] = c;
            if (i == N - 1 && col == M - 1) {
              a.loss64[b] = c;
              a.loss[b] = (float)c;
            }
          }
        } else if (ok) {
          const double z = ((rnm + (double)dv[u]) - (rv[u] + c)) * k2;
          Erow[M - 1 - col] = hw_exp2((float)z);
        }
      }

      // Hand lane 63's cells (row r0+63, columns t0+u-63) to the band below.
      if (!last_in_seg) {
        if (lane == 63) {
#pragma unroll
          for (int u = 0; u < kCH; ++u) ring[w][(t0 + u - 63) & (kRing - 1)] = bottom[u];
        }
      } else if (produce_global) {
        if (lane == 63) {
#pragma unroll
          for (int u = 0; u < kCH; ++u) {
            const int64_t col = t0 + u - 63;
            if (col >= 0 && col < M) Hout[col] = bottom[u];
          }
          if (((q + 1) % kPub) == 0 || q == qcount - 1) {
            int64_t done = t0 + kCH - 63;
            done = done < 0 ? 0 : imin64(done, M);
            __hip_atomic_store(prog_out, (unsigned)done, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_dp(const DPArgs& a, bool reverse, bool fused, hipStream_t s) {
  if (fused) return hipErrorNotSupported;
  const unsigned grid = (unsigned)a.B * (unsigned)a.nseg;
  if (reverse)
    hipLaunchKernelGGL(k_dp_unfused<true>, dim3(grid), dim3(kBandsPerWG * 64), 0, s, a);
  else
    hipLaunchKernelGGL(k_dp_unfused<false>, dim3(grid), dim3(kBandsPerWG * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdtw

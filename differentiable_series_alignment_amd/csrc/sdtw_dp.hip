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
#include "sdtw_dp_common.h"

namespace sdtw {

__global__ void k_zero_u32(unsigned* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Sixteen steps of one band.  MASK: the chunk contains steps with column < 0
// (only the first 64 steps do); those cells are the left boundary, +inf
// except the corner R[-1,-1] = 0 handled through the initial state.
template <bool REV, bool MASK>
__device__ __forceinline__ void band_chunk(double& cur, double& up, const double (&top)[16],
                                           const float (&dn)[16], const double (&rn)[16],
                                           double (&bottom)[16], int64_t t0, int lane,
                                           bool row_ok, double k2, double xnm,
                                           float* __restrict__ dsk, double* __restrict__ rsk,
                                           const LaneCursor& cu) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t t = t0 + u;
    const double d = row_ok ? (double)dn[u] * k2 : 0.0;
    const double upn = wave_shr1(cur, top[u]);
    const double diag = up;
    up = upn;
    double c = softmin2_cell(diag, upn, cur, d);
    if (MASK) c = (t - lane < 0) ? kBig : c;
    cur = c;
    bottom[u] = c;
    const int64_t e = cu.base + t * cu.dir;
    if (!REV) {
      __builtin_nontemporal_store(c, rsk + e);
    } else {
      // ln E = (R[N-1,M-1] + Dist - R - R') / g, i.e. in base-2 units
      // log2 E = Xnm + d - X - X'; the exponential is taken last.
      __builtin_nontemporal_store(hw_exp2((float)((xnm + d) - (rn[u] + c))), dsk + e);
    }
  }
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

  const int64_t N = a.N, M = a.M, S = a.S;
  const int band = seg * W + w;
  const int nb_seg = min(W, a.nbands - seg * W);
  const bool active = w < nb_seg;
  const int64_t r0 = (int64_t)(active ? band : 0) * 64;
  const int64_t i = r0 + lane;                        // sweep-space row
  const bool row_ok = active && i < N;
  const int qcount = (int)(sweep_steps(M) / kCH);
  const int qtot = qcount + kLag * (nb_seg - 1);
  const bool last_in_seg = (w == nb_seg - 1);
  const bool produce_global = active && last_in_seg && (seg + 1 < a.nseg);
  const bool consume_global = active && (w == 0) && (seg > 0);

  unsigned* prog_in = a.ctrl + 2 + (int64_t)b * a.nseg + (seg > 0 ? seg - 1 : 0);
  unsigned* prog_out = a.ctrl + 2 + (int64_t)b * a.nseg + seg;
  const double* Hin = a.H + ((int64_t)b * a.nseg + (seg > 0 ? seg - 1 : 0)) * M;
  double* Hout = a.H + ((int64_t)b * a.nseg + seg) * M;

  const LaneCursor cu = lane_cursor(REV, b, i, lane, N, M, a.nbands, S);
  float* dsk = a.dsk;
  double* rsk = a.R;
  const double k2 = a.k2;
  const double xnm = REV ? a.loss64[b] : 0.0;

  // Boundary: R[-1,-1] = 0 reaches the first row's first cell as the
  // diagonal input of step 0 (lane 0 of band 0); all else is +inf.
  double cur = kBig;
  double up = (lane == 0 && r0 == 0) ? 0.0 : kBig;
  unsigned avail = 0;

  // Position of the final cell (forward sweep): row N-1, column M-1.
  const int64_t lastrow = N - 1;
  const bool has_last = !REV && active && (lastrow >> 6) == band;
  const int64_t tlast = M - 1 + (lastrow & 63);
  const int qlast = (int)(tlast / kCH), ulast = (int)(tlast % kCH);

  // Every global access below is unconditional (padding cells have storage)
  // and the data of chunk q+1 is requested while chunk q computes, so memory
  // latency stays off the per-step dependency chain.
  float dn[kCH];
  double rn[kCH];
  double tn[kCH];  // raw top-row values from the segment above (masked at use)
#define SDTW_LOAD_CHUNK(qq, D_, R_)                                       \
  {                                                                       \
    const int64_t t0n = (int64_t)(qq) * kCH;                              \
    _Pragma("unroll") for (int u = 0; u < kCH; ++u) {                     \
      const int64_t e = cu.base + (t0n + u) * cu.dir;                     \
      D_[u] = dsk[e];                                                     \
      if (REV) R_[u] = rsk[e];                                            \
    }                                                                     \
  }
  // Wait (bounded) until the segment above has published `need` columns.
#define SDTW_AWAIT(need_)                                                 \
  {                                                                       \
    const unsigned need = (unsigned)(need_);                              \
    if (avail < need) avail = await_progress(prog_in, need);              \
  }
#define SDTW_LOAD_TOP(qq, T_)                                             \
  {                                                                       \
    const int64_t t0n = (int64_t)(qq) * kCH;                              \
    _Pragma("unroll") for (int u = 0; u < kCH; ++u) {                     \
      const int64_t col = t0n + u;                                        \
      T_[u] = Hin[col < M ? col : M - 1];                                 \
    }                                                                     \
  }

  if (active) SDTW_LOAD_CHUNK(0, dn, rn);
  if (consume_global) {
    SDTW_AWAIT(imin64(M, kCH + kSlack));
    SDTW_LOAD_TOP(0, tn);
  }
  // Drain the first requests here, so that inside the loop the only loads
  // in flight are the ones for the next chunk (the counter-based waits are
  // then exact instead of covering those as well).
  __builtin_amdgcn_s_waitcnt(0);

  for (int Q = 0; Q < qtot; ++Q) {
    const int q = Q - kLag * w;
    if (active && q >= 0 && q < qcount) {
      const int64_t t0 = (int64_t)q * kCH;
      // Requests for chunk q+1 go out first, into fresh registers.
      float dn2[kCH];
      double rn2[kCH];
      double tn2[kCH];
      const bool more = q + 1 < qcount;
      if (more) {
        SDTW_LOAD_CHUNK(q + 1, dn2, rn2);
        if (consume_global) {
          SDTW_AWAIT(imin64(M, t0 + 2 * kCH));
          SDTW_LOAD_TOP(q + 1, tn2);
        }
      }
      double top[kCH];
      if (r0 == 0) {
#pragma unroll
        for (int u = 0; u < kCH; ++u) top[u] = kBig;
      } else if (!consume_global) {
#pragma unroll
        for (int u = 0; u < kCH; ++u) top[u] = ring[w - 1][(t0 + u) & (kRing - 1)];
      } else {
#pragma unroll
        for (int u = 0; u < kCH; ++u) top[u] = tn[u];
      }

      double bottom[kCH];
      if (t0 < 64)
        band_chunk<REV, true>(cur, up, top, dn, rn, bottom, t0, lane, row_ok, k2, xnm,
                              dsk, rsk, cu);
      else
        band_chunk<REV, false>(cur, up, top, dn, rn, bottom, t0, lane, row_ok, k2, xnm,
                               dsk, rsk, cu);

      if (has_last && q == qlast) {
        double v = 0.0;
#pragma unroll
        for (int u = 0; u < kCH; ++u) v = (u == ulast) ? bottom[u] : v;
        if (lane == (int)(lastrow & 63)) {
          a.loss64[b] = v;
          a.loss[b] = (float)(v * a.g_ln2);
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
      // Rotate the prefetched chunk in; its loads were issued a chunk ago.
      if (more) {
#pragma unroll
        for (int u = 0; u < kCH; ++u) {
          dn[u] = dn2[u];
          if (REV) rn[u] = rn2[u];
          if (consume_global) tn[u] = tn2[u];
        }
      }
    }
    __syncthreads();
  }
#undef SDTW_LOAD_CHUNK
#undef SDTW_AWAIT
#undef SDTW_LOAD_TOP
  release_ctrl(a.ctrl, (int64_t)a.B * a.nseg);
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

__global__ void k_zero_f32(float* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_dp(const DPArgs& a, bool reverse, bool fused, hipStream_t s) {
  if (fused) return launch_dp_fused(a, reverse, s);
  const unsigned grid = (unsigned)a.B * (unsigned)a.nseg;
  if (reverse)
    hipLaunchKernelGGL(k_dp_unfused<true>, dim3(grid), dim3(kBandsPerWG * 64), 0, s, a);
  else
    hipLaunchKernelGGL(k_dp_unfused<false>, dim3(grid), dim3(kBandsPerWG * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdtw

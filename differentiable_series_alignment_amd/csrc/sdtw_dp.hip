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
//    to fp64 differences (see softmin2_cell);
//  - the kBandsPerWG band waves of a workgroup run decoupled, each at its own
//    pace, chunk by chunk (16 steps); band w reads its top row from an LDS
//    ring that band w-1's lane 63 fills, with written/released column
//    counters instead of barriers;
//  - consecutive workgroups of one pair ("segments") hand the bottom row of
//    the segment over through global memory; one extra wave per workgroup
//    does that copying and signalling, so band waves only ever wait on LDS;
//    workgroups take tickets in arrival order and a segment only waits on a
//    smaller ticket, so the wait always ends.
//
// The reverse sweep runs the same recurrence on both sequences reversed,
// which yields R'[i,j], the soft-DTW value of the suffix alignment from
// (i,j) to (N-1,M-1) that includes Dist[i,j].  Splitting every alignment
// path at (i,j) gives the alignment matrix in log space,
//   ln E[i,j] = (R[N-1,M-1] + Dist[i,j] - R[i,j] - R'[i,j]) / g,
// exponentiated only at the end (the log-space backward with a final exp of
// the review page "SoftDTW-CUDA-Torch", section "Proposed method").  The two
// sweeps are independent, so one launch runs both at once: the forward
// sweep keeps X = R log2(e)/g, the reverse sweep keeps T' = (R' - Dist)
// log2(e)/g, its soft-minimum part, and E = 2^(Xnm - X - T') is formed
// later, by the chain-rule kernel.
#include "sdtw_dp_common.h"

namespace sdtw {

__global__ void k_zero_u32(unsigned* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Sixteen steps of one band.  MASK: the chunk contains steps with column < 0
// (only the first 64 steps do); those cells are the left boundary.  Giving
// them the distance kBig makes every such state at least kBig (the +inf
// stand-in) without touching the dependency chain; the corner R[-1,-1] = 0
// enters through the initial state of lane 0 of the first band.  Cells past
// the last column or below the last row compute unused values in padding
// storage; no real cell depends on them.  The forward sweep stores X, the
// reverse sweep its soft-minimum part T'.  EFORM (reverse sweep after a
// completed forward): the cell's X comes in xn and the reverse sweep stores
// E = 2^(Xnm - X - T') in place of its distance (ep), 0 outside the grid
// (sweep column t0 + u - lane outside 0..M-1, or a padding row).  NT: the
// states go out as nontemporal stores (see launch_dp_both).
template <bool REV, bool MASK, bool EFORM = false, bool NT = true>
__device__ __forceinline__ void band_chunk(double& cur, double& up, const double (&top)[16],
                                           const float (&dn)[16], double (&bottom)[16],
                                           int t0, int lane, double k2,
                                           double* __restrict__ sp,
                                           const double (&xn)[EFORM ? 16 : 1],
                                           float* __restrict__ ep, double xnm, bool row_ok,
                                           int M) {
  constexpr int dir = REV ? -64 : 64;
  // Steps 8..15 address from a second base so every store of the chunk is
  // base + immediate offset.
  double* const sp8 = sp + 8 * dir;
  float* const ep8 = ep + 8 * dir;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    double d = (double)dn[u] * k2;
    if (MASK) d = (t0 + u < lane) ? kBig : d;
    const double upn = wave_shr1(cur, top[u]);
    double t;
    const double c = softmin2_cell(up, upn, cur, d, t);
    up = upn;
    cur = c;
    bottom[u] = c;
    if (EFORM) {
      const int jc = t0 + u - lane;
      const bool ok = row_ok && jc >= 0 && jc < M;
      const float e = ok ? align_entry(xnm, xn[EFORM ? u : 0], t) : 0.f;
      __builtin_nontemporal_store(e, (u < 8 ? ep : ep8) + (u & 7) * dir);
    } else {
      double* const dst = (u < 8 ? sp : sp8) + (u & 7) * dir;
      if (NT)
        __builtin_nontemporal_store(REV ? t : c, dst);
      else
        *dst = REV ? t : c;
    }
  }
}

// s_waitcnt operand (gfx9 layout: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in [15:14]) that waits until at most 16 vector-memory
// operations are outstanding and does not wait on the other counters.
constexpr int kWaitVm16 = (1 << 14) | (7 << 4) | (15 << 8);

// Loads of one chunk's distances (16 steps from `off`), two bases as above.
template <bool REV>
__device__ __forceinline__ void load_chunk(const float* dbase, int64_t off, float (&dn)[16]) {
  constexpr int dir = REV ? -64 : 64;
  const float* d0 = dbase + off;
  const float* d8 = d0 + 8 * dir;
#pragma unroll
  for (int u = 0; u < 16; ++u) dn[u] = (u < 8 ? d0 : d8)[(u & 7) * dir];
}
// The same for the forward states X the E-forming reverse sweep reads.
template <bool REV>
__device__ __forceinline__ void load_xchunk(const double* xbase, int64_t off, double (&xn)[16]) {
  constexpr int dir = REV ? -64 : 64;
  const double* x0 = xbase + off;
  const double* x8 = x0 + 8 * dir;
#pragma unroll
  for (int u = 0; u < 16; ++u) xn[u] = (u < 8 ? x0 : x8)[(u & 7) * dir];
}

// One band of one pair, swept column chunk by column chunk.  The band's top
// row comes from LDS ring `w`: the previous band's bottom row, the row the
// segment's I/O wave copies in, or (first band of a pair) a ring the
// workgroup filled with kBig and marked complete.  Its bottom row goes to
// LDS ring `w + 1` when a band or the segment's I/O wave reads it.
//
// The next chunk's top entries are read at the end of each chunk, after the
// ring's written count; if that count already covers them (the usual case:
// a band runs a little slower than the band above it), the chunk starts
// without touching LDS, otherwise it polls and reads them again.  LDS
// operations of one wave complete in issue order, so entries read after a
// count that covers them are the published ones.
template <bool REV, bool EFORM = false, bool NT = true>
__device__ __forceinline__ void band_sweep(const DPArgs& a, int b, int seg, int w, int nb_seg,
                                           double (*ring)[kRingC + kCH], unsigned* wr,
                                           unsigned* rd, int lane) {
  constexpr int W = kBandsPerWG;
  const int64_t N = a.N, M = a.M, S = a.S;
  const int band = seg * W + w;
  const int64_t r0 = (int64_t)band * 64;
  const int64_t i = r0 + lane;                         // sweep-space row
  const int qcount = (int)(sweep_steps(M) / kCH);
  const bool out_used = (w + 1 < nb_seg) || (seg + 1 < a.nseg);
  const unsigned Mu = (unsigned)M;

  const LaneCursor cu = lane_cursor(REV, b, i, lane, N, M, a.nbands, S);
  const float* const dbase = a.dsk + cu.base;
  // EFORM: X of the same cells (same element index), E over the distances.
  double* const sbase = EFORM ? nullptr : (REV ? a.R2 : a.R) + cu.base;
  const double* const xsrc = EFORM ? a.R + cu.base : nullptr;
  float* const ebase = EFORM ? a.dsk + cu.base : nullptr;
  const double xnm = EFORM ? a.loss64[b] : 0.0;
  const bool row_ok = i < N;
  const double k2 = a.k2;

  // Final cell (forward sweep): row N-1, column M-1.
  const int64_t lastrow = N - 1;
  const bool has_last = !REV && (lastrow >> 6) == band;
  const int64_t tlast = M - 1 + (lastrow & 63);
  const int qlast = (int)(tlast / kCH), ulast = (int)(tlast % kCH);

  double cur = kBig;
  double up = (band == 0 && lane == 0) ? 0.0 : kBig;
  unsigned seen_rd = 0;

  // Chunk inputs alternate between two register sets: chunk q computes from
  // one while the requests for chunk q+1 fill the other.
  float dnA[kCH], dnB[kCH];
  double xA[EFORM ? kCH : 1], xB[EFORM ? kCH : 1];
  load_chunk<REV>(dbase, 0, dnA);
  if constexpr (EFORM) load_xchunk<REV>(xsrc, 0, xA);
  // Top entries of the first chunk and the count they were read under.
  double top[kCH];
  unsigned seen_wr = __hip_atomic_load(&wr[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int u = 0; u < kCH; ++u) top[u] = ring[w][u];
  __builtin_amdgcn_s_waitcnt(0);

  auto chunk = [&](int q, const float (&dn)[kCH], float (&dn2)[kCH],
                   const double (&xn)[EFORM ? kCH : 1], double (&xn2)[EFORM ? kCH : 1]) {
    const int t0 = q * kCH;
    // This chunk's loads were issued before the previous chunk's 16 stores;
    // the vector-memory counter retires in issue order, so allowing 16
    // operations in flight completes the loads and leaves the stores going.
    __builtin_amdgcn_s_waitcnt(kWaitVm16);
    // Top row, columns t0 .. t0+15 (entries past M are never used).
    const unsigned need = (unsigned)t0 + kCH < Mu ? (unsigned)t0 + kCH : Mu;
    if (seen_wr < need) {
      seen_wr = lds_wait_ge(&wr[w], need);
#pragma unroll
      for (int u = 0; u < kCH; ++u) top[u] = ring[w][(t0 + u) & (kRingC - 1)];
    }
    // Unconditional (the last chunk re-reads its own cells), so the
    // compiler's wait bookkeeping stays exact across the loop.
    const int64_t noff = (int64_t)(q + 1 < qcount ? t0 + kCH : t0) * cu.dir;
    load_chunk<REV>(dbase, noff, dn2);
    double bottom[kCH];
    if constexpr (EFORM) {
      load_xchunk<REV>(xsrc, noff, xn2);
      float* ep = ebase + (int64_t)t0 * cu.dir;
      if (t0 < 64)
        band_chunk<REV, true, true>(cur, up, top, dn, bottom, t0, lane, k2, nullptr, xn, ep,
                                    xnm, row_ok, (int)M);
      else
        band_chunk<REV, false, true>(cur, up, top, dn, bottom, t0, lane, k2, nullptr, xn, ep,
                                     xnm, row_ok, (int)M);
    } else {
      double* sp = sbase + (int64_t)t0 * cu.dir;
      if (t0 < 64)
        band_chunk<REV, true, false, NT>(cur, up, top, dn, bottom, t0, lane, k2, sp, xn,
                                         nullptr, 0.0, true, 0);
      else
        band_chunk<REV, false, false, NT>(cur, up, top, dn, bottom, t0, lane, k2, sp, xn,
                                          nullptr, 0.0, true, 0);
    }

    if (has_last && q == qlast) {
      double v = 0.0;
#pragma unroll
      for (int u = 0; u < kCH; ++u) v = (u == ulast) ? bottom[u] : v;
      if (lane == (int)(lastrow & 63)) {   // device-coherent (see release_ctrl)
        __hip_atomic_store(a.loss64 + b, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.loss + b, (float)(v * a.g_ln2), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // Next chunk's top entries, read after the count (see above), and ahead
    // of this chunk's LDS writes so that they return first.  Their slots are
    // not released yet, so the band above cannot overwrite them.
    seen_wr = __hip_atomic_load(&wr[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int u = 0; u < kCH; ++u) top[u] = ring[w][(t0 + kCH + u) & (kRingC - 1)];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // The top entries of this chunk have been read: release them.
    if (lane == 0) lds_publish(&rd[w], need);
    // Lane 63's cells (row r0+63, columns t0+u-63) go to the row below.
    if (out_used) {
      const int cmax = t0 + kCH - 1 - 63;          // newest column of this chunk
      if (cmax >= kRingC) {
        const unsigned need_rd = (unsigned)(cmax - kRingC + 1);
        if (seen_rd < need_rd) seen_rd = lds_wait_ge(&rd[w + 1], need_rd);
      }
      if (lane == 63) {
        // Columns t0-63 .. t0-48 occupy slots s .. s+15 with s = 1 (mod 16),
        // so the run is contiguous in the padded ring row and only s = 241
        // spills into the pad, whose one slot (256) mirrors slot 0.  Slots
        // of negative columns (first chunks) belong to columns not yet
        // published, so writing them is harmless.
        const int s0 = (t0 + kRingC - 63) & (kRingC - 1);
        double* rw = &ring[w + 1][s0];
#pragma unroll
        for (int u = 0; u < kCH; ++u) rw[u] = bottom[u];
        if (s0 + kCH > kRingC) ring[w + 1][0] = bottom[kRingC - s0];
        const int done = t0 + kCH - 63;
        lds_publish(&wr[w + 1], done <= 0 ? 0u : ((unsigned)done < Mu ? (unsigned)done : Mu));
      }
    }
  };

  for (int q = 0; q < qcount; q += 2) {
    chunk(q, dnA, dnB, xA, xB);
    if (q + 1 < qcount) chunk(q + 1, dnB, dnA, xB, xA);
  }
}

// Both sweeps in one launch (a.sweeps == kSweepsBoth), or one of them.  With
// both, tickets alternate between the sweeps, so the forward and reverse
// workgroups of a pair start together; within a sweep a segment waits only
// on the previous segment, which holds a smaller ticket.  Control words: [0]
// ticket, [1] finished workgroups, [2 + sweep*B*nseg + b*nseg + s] columns
// published by segment s of pair b; H holds one bottom row per (sweep, pair,
// segment).  The E-forming reverse sweep (kSweepReverseE) runs once per
// forward: its last workgroup sets *a.eflag, and a launch that finds the
// flag set (a repeated backward) leaves E as it is.
// ERV: the E-forming reverse sweep (its own instance: the forward states it
// reads take registers the other sweeps do not need).  NT: nontemporal
// state stores.
template <bool ERV, bool NT = true>
__global__ __launch_bounds__((kBandsPerWG + 1) * 64) void k_dp_unfused(DPArgs a) {
  constexpr int W = kBandsPerWG;
  __shared__ double ring[W + 1][kRingC + kCH];   // + pad, see band_sweep
  __shared__ unsigned wr[W + 1], rd[W + 1];
  __shared__ unsigned s_ticket, s_skip;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  constexpr bool eform = ERV;
  if (threadIdx.x == 0) {
    s_ticket = atomicAdd(&a.ctrl[0], 1u);
    s_skip = eform ? __hip_atomic_load(a.eflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0u;
    launch_shared_init(a);
  }
  __syncthreads();
  const unsigned ticket = s_ticket;
  const bool both = !ERV && a.sweeps == kSweepsBoth;
  const int rev = both ? (int)(ticket & 1u) : (eform ? 1 : 0);
  const unsigned rest = both ? ticket >> 1 : ticket;
  const int seg = (int)(rest / (unsigned)a.B);
  const int b = (int)(rest % (unsigned)a.B);
  // The first band of a pair reads its top row (the +inf boundary) from
  // ring 0, filled with kBig and marked complete.
  if (threadIdx.x < W + 1) {
    wr[threadIdx.x] = (seg == 0 && threadIdx.x == 0) ? (unsigned)a.M : 0u;
    rd[threadIdx.x] = 0u;
  }
  if (seg == 0)
    for (int k = threadIdx.x; k < kRingC + kCH; k += blockDim.x) ring[0][k] = kBig;
  __syncthreads();
  const int nb_seg = min(W, a.nbands - seg * W);
  const int64_t per_sweep = (int64_t)a.B * a.nseg;

  if (s_skip) {
    // E already formed for this forward: nothing to do.
  } else if (w == W) {
    const int64_t pb = rev * per_sweep + (int64_t)b * a.nseg;
    const int64_t sin = pb + (seg > 0 ? seg - 1 : 0), sout = pb + seg;
    GlobalRow gr{0u, nullptr, nullptr};
    gr.valid_in = gr.valid_out = a.hvalid != 0;
    segment_io_wave(seg > 0, seg + 1 < a.nseg, a.ctrl + 2 + sin, a.ctrl + 2 + sout,
                    a.H + sin * a.M, a.H + sout * a.M, ring[0], &wr[0], &rd[0], ring[W],
                    &wr[W], &rd[W], (unsigned)a.M, lane, gr);
  } else if (w < nb_seg) {
    if constexpr (ERV)
      band_sweep<true, true>(a, b, seg, w, nb_seg, ring, wr, rd, lane);
    else if (rev)
      band_sweep<true, false, NT>(a, b, seg, w, nb_seg, ring, wr, rd, lane);
    else
      band_sweep<false, false, NT>(a, b, seg, w, nb_seg, ring, wr, rd, lane);
  }
  const bool last = release_ctrl(a.ctrl, 2 * per_sweep, true);
  if (last && eform && !s_skip && threadIdx.x == 0)
    __hip_atomic_store(a.eflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Control words to zero and hand-off entries to kHEmpty, in one launch.
__global__ void k_clear(unsigned* zero, int64_t nzero, uint64_t* empty, int64_t nempty) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nzero; i += stride)
    zero[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nempty; i += stride)
    empty[i] = kHEmpty;
}

hipError_t launch_clear(unsigned* zero, int64_t nzero, double* empty, int64_t nempty,
                        hipStream_t s) {
  const int64_t n = nzero > nempty ? nzero : nempty;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  TimedLaunch timed_("clear", s);
  hipLaunchKernelGGL(k_clear, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                     zero, nzero, reinterpret_cast<uint64_t*>(empty), nempty);
  return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimedLaunch timed_("zero_u32", s);
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

__global__ void k_fill_u32(unsigned* p, int64_t n, unsigned v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(unsigned* p, int64_t n, unsigned v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimedLaunch timed_("fill_u32", s);
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

__global__ void k_zero_f32(float* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimedLaunch timed_("zero_f32", s);
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// The states of both sweeps go out as ordinary stores when they fit in the
// GPU's last-level cache with room to spare (MI355X: 256 MiB of Infinity
// Cache), so the chain rule that reads them next finds them there: B=32,
// N=M=512 (151 MB of states) row pass 60.9 -> 55.4 us, sweeps unchanged.
// Larger arrays go out nontemporal: with ordinary stores B=32, N=M=1024,
// D=128 (570 MB) took 270 against 216 us for the sweeps and 189 against
// 174 us for the row pass.
constexpr size_t kStateCacheBytes = size_t(160) << 20;

hipError_t launch_dp_both(const DPArgs& a, hipStream_t s) {
  const unsigned grid = (a.sweeps == kSweepsBoth ? 2u : 1u) * (unsigned)a.B * (unsigned)a.nseg;
  TimedLaunch timed_(a.sweeps == kSweepsBoth ? "dp_both"
                     : a.sweeps == kSweepForward ? "dp_forward" : "dp_reverse_e", s);
  const size_t state_bytes =
      2 * (size_t)band_array_elems((int64_t)a.B * a.nbands, a.S, a.M) * sizeof(double);
  if (a.sweeps == kSweepReverseE)
    hipLaunchKernelGGL(k_dp_unfused<true>, dim3(grid), dim3((kBandsPerWG + 1) * 64), 0, s, a);
  else if (a.sweeps == kSweepsBoth && state_bytes <= kStateCacheBytes)
    hipLaunchKernelGGL((k_dp_unfused<false, false>), dim3(grid), dim3((kBandsPerWG + 1) * 64), 0,
                       s, a);
  else
    hipLaunchKernelGGL((k_dp_unfused<false, true>), dim3(grid), dim3((kBandsPerWG + 1) * 64), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace sdtw

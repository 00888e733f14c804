// Pieces shared by the unfused and fused wavefront kernels: chunking
// constants, the control words of a sweep, and the per-lane band cursor.
#pragma once
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

constexpr int kCH = 16;                      // steps per chunk
constexpr int kLag = 2 + 62 / kCH;           // chunks between adjacent bands
constexpr int kRing = 128;                   // LDS ring columns per boundary
constexpr int kPub = 4;                      // chunks between global publishes
constexpr int kSlack = 96;                   // extra columns awaited at start
constexpr uint32_t kSpinCap = 1u << 25;      // polls before a wait gives up
static_assert(kRing >= (kLag + 3) * kCH, "LDS ring too small");
static_assert(kCH == 16, "band_chunk unrolls 16 steps");

// Control words of one sweep: [0] ticket, [1] finished workgroups,
// [2 + b*nseg + s] columns published by segment s of pair b.  The last
// workgroup to finish returns them to zero, so the next launch on the same
// workspace starts clean without a separate clearing launch (every other
// workgroup has stopped touching them once it has counted itself finished).
__device__ __forceinline__ void release_ctrl(unsigned* ctrl, int64_t nprog) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned done = __hip_atomic_fetch_add(&ctrl[1], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      for (int64_t k = 0; k < nprog; ++k)
        __hip_atomic_store(&ctrl[2 + k], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl[1], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Bounded wait until *prog >= need (columns published by the segment above).
// The polls are relaxed; one agent-scope acquire fence follows the poll that
// succeeds, so waiting does not invalidate caches on every poll.  The producer
// holds a smaller ticket and is running, so it publishes within one sweep; the
// cap only guarantees that every wave exits even if that ever failed (the
// result would be garbage, never a hang).  Returns the value to record as
// available.
__device__ __forceinline__ unsigned await_progress(const unsigned* prog, unsigned need) {
  unsigned v = 0;
  for (uint32_t spin = 0; spin < kSpinCap; ++spin) {
    v = __hip_atomic_load(prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= need) break;
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return v < need ? need : v;
}

// Per-lane view of one band of a band-step array: the element a sweep step t
// touches is base[t * dir] (dir = +64 forward, -64 reverse).
struct LaneCursor {
  int64_t base;  // element index at t = 0
  int64_t dir;
};

// Storage row of sweep row i: the forward sweep's rows are the original rows;
// the reverse sweep's row i is original row N-1-i.  Sweep rows past the grid
// (the padding of the last band) map onto the padding rows of storage, so
// stores of padding cells never touch a real cell.
__device__ __forceinline__ LaneCursor lane_cursor(bool rev, int64_t b, int64_t i,
                                                  int lane, int64_t N, int64_t M,
                                                  int nbands, int64_t S) {
  LaneCursor c;
  if (!rev) {
    const int64_t r = i;  // lane == r % 64; cell (r, t - lane) is at step t + off
    c.base = ((b * nbands + (r >> 6)) * S + kSkewOff) * 64 + (r & 63);
    c.dir = 64;
  } else {
    const int64_t r = i < N ? N - 1 - i : i;
    const int64_t l = r & 63;
    // cell (r, M-1-(t-lane)) sits at step M-1-t+lane+l+off
    c.base = ((b * nbands + (r >> 6)) * S + (M - 1 + lane + l + kSkewOff)) * 64 + l;
    c.dir = -64;
  }
  return c;
}

}  // namespace sdtw

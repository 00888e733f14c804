// Pieces shared by the unfused and fused wavefront kernels: chunking
// constants, the control words of a sweep, and the per-lane band cursor.
#pragma once
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

constexpr int kCH = 16;                      // steps per chunk
constexpr uint32_t kSpinCap = 1u << 25;      // idle polls of a global row before a wait gives up
constexpr uint32_t kLdsSpinCap = 1u << 22;   // polls of an LDS counter before a wait gives up
static_assert(kCH == 16, "band_chunk unrolls 16 steps");

// Wait limits and the error word.  Every wait below is a bounded poll: if
// the value it waits for does not come within a cap of polls (about 0.1 s
// for LDS counters, seconds for global rows), it gives up so that every wave
// still exits, and records that in the workspace's error word (an
// agent-scope atomic OR, waited for, so the launch's last workgroup sees
// it).  That workgroup then sets the launch's outputs to NaN (release_ctrl),
// and sdtw_workspace_status reports the error on the host.  A nonzero
// DPArgs::wait_cap replaces both caps (a test hook).
//
// What the waits and the end of the launch need (the error word, the cap,
// the outputs to poison) is copied into LDS by thread 0 at the start of a
// launch (launch_shared_init, before the kernel's first barrier), so no
// register holds it across the sweep: waits read the cap only once they
// have to wait.
struct LaunchShared {
  unsigned* err;
  unsigned cap;
  float* loss;
  double* loss64;
  float* gx;
  float* gy;
  float* align;
  int64_t nb, nx, ny, na;   // element counts of loss, gx, gy, align
};
__device__ __forceinline__ LaunchShared& launch_shared() {
  __shared__ LaunchShared ls;
  return ls;
}
__device__ __forceinline__ void launch_shared_init(const DPArgs& a) {
  LaunchShared& ls = launch_shared();
  ls.err = a.err;
  ls.cap = a.wait_cap;
  ls.loss = a.loss;
  ls.loss64 = a.loss64;
  ls.gx = a.gx;
  ls.gy = a.gy;
  ls.align = a.align;
  ls.nb = a.B;
  ls.nx = (int64_t)a.B * a.N * a.D;
  ls.ny = (int64_t)a.B * a.M * a.D;
  ls.na = (int64_t)a.B * a.N * a.M;
}
__device__ __forceinline__ uint32_t lds_cap() {
  const unsigned c = launch_shared().cap;
  return c ? c : kLdsSpinCap;
}
__device__ __forceinline__ uint32_t glob_cap() {
  const unsigned c = launch_shared().cap;
  return c ? c : kSpinCap;
}
__device__ __forceinline__ void note_giveup() {
  unsigned* err = launch_shared().err;
  if (err) {
    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// NaN over every output the launch writes (the loss and the fp64 final
// state that later launches start from; gradients and the alignment matrix
// of a reverse sweep), by the threads of one workgroup.
__device__ __forceinline__ void poison_outputs() {
  const LaunchShared& ls = launch_shared();
  const float qnan = __builtin_nanf("");
  const int64_t t0 = threadIdx.x, nt = blockDim.x;
  for (int64_t i = t0; i < ls.nb; i += nt) {
    if (ls.loss) ls.loss[i] = qnan;
    if (ls.loss64) ls.loss64[i] = __builtin_nan("");
  }
  if (ls.gx)
    for (int64_t i = t0; i < ls.nx; i += nt) ls.gx[i] = qnan;
  if (ls.gy)
    for (int64_t i = t0; i < ls.ny; i += nt) ls.gy[i] = qnan;
  if (ls.align)
    for (int64_t i = t0; i < ls.na; i += nt) ls.align[i] = qnan;
}

// Control words of one sweep: [0] ticket, [1] finished workgroups,
// [2 + b*nseg + s] columns published by segment s of pair b.  The last
// workgroup to finish returns them to zero, so the next launch on the same
// workspace starts clean without a separate clearing launch (every other
// workgroup has stopped touching them once it has counted itself finished),
// and, if any wait of the launch gave up, poisons the launch's outputs.
// Returns true in the last workgroup (every other one has finished).
//
// Ordering without cache maintenance (coherent = true): every wave waits
// for its own memory operations before the barrier, and only then is the
// workgroup counted, with a relaxed device-coherent atomic.  The control
// words, the hand-off rows and the error word are only ever accessed with
// device-coherent atomics, and every output the last workgroup may poison
// is written with device-coherent stores, so what another workgroup did
// before it counted itself is in memory, and the poison (an ordinary store
// in the last workgroup's cache) is written back after it.  An acquire or
// release at device scope instead writes back or invalidates the whole L2
// of the XCD, once per workgroup: 32x4096x1000 sweeps 916 -> 831 us without
// it.  coherent = false keeps that path, for a launch whose outputs are
// written with ordinary stores (the fused reverse with an alignment-matrix
// output, whose scattered stores would cost more as device-coherent ones).
__device__ __forceinline__ bool release_ctrl(unsigned* ctrl, int64_t nprog, bool coherent) {
  __shared__ unsigned s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned done =
        coherent ? __hip_atomic_fetch_add(&ctrl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : __hip_atomic_fetch_add(&ctrl[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == gridDim.x - 1;
    if (s_last) {
      for (int64_t k = 0; k < nprog; ++k)
        __hip_atomic_store(&ctrl[2 + k], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (coherent)
        __hip_atomic_store(&ctrl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_store(&ctrl[1], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  unsigned* const err = launch_shared().err;
  if (s_last && err &&
      (coherent ? __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                : __hip_atomic_load(err, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)) != 0u)
    poison_outputs();
  return s_last;
}

// Hand-off stress (debug builds only: SDTW_STRESS=1, built as
// libsdtw_stress.so).  Every producer's publish, every consumer's wait and
// every pass of a hand-off wave first sleeps a pseudo-random time: mostly
// 0-3 sleeps of 8 x 64 clocks, one time in eight up to 63 of them (about
// 13 us).  The hash mixes the clock with the site, workgroup and wave, so
// producers and consumers drift against each other differently on every
// run; results must not change, only timings.  In normal builds it is empty.
#ifndef SDTW_STRESS
#define SDTW_STRESS 0
#endif
__device__ __forceinline__ void stress_delay(unsigned site) {
#if SDTW_STRESS
  const uint64_t t = __builtin_readcyclecounter();
  uint32_t h = (uint32_t)t ^ (uint32_t)(t >> 32) ^ (site * 0x9E3779B9u) ^
               (blockIdx.x * 0x85EBCA6Bu) ^ ((threadIdx.x >> 6) * 0xC2B2AE35u);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  h = __builtin_amdgcn_readfirstlane(h);
  const uint32_t n = (h & 7u) == 0u ? (h >> 3) & 63u : (h >> 3) & 3u;
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
#else
  (void)site;
#endif
}

// ---------------------------------------------------------------------------
// Decoupled bands.  Inside a workgroup every band wave runs at its own pace;
// the row a band hands to the band below travels through an LDS ring of
// kRingC columns with two counters: wr = columns written (all columns below
// it are valid), rd = columns released by the reader (their slots may be
// overwritten).  LDS operations of one wave are performed in issue order, so
// a counter written after the ring entries never runs ahead of them, and a
// read issued after the counter was seen never sees older entries.
// ---------------------------------------------------------------------------
constexpr int kRingC = 256;                  // columns per LDS ring (power of 2)

// Bounded wait until *p >= need; returns the last value read (>= need unless
// the cap was hit: then the give-up is recorded (note_giveup) and the caller
// proceeds on stale data rather than hang; the launch's outputs become NaN).
__device__ __forceinline__ unsigned lds_wait_ge(const unsigned* p, unsigned need) {
  stress_delay(1);
  unsigned v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (v >= need) return v;
  const uint32_t cap = lds_cap();
  for (uint32_t spin = 0; v < need; ++spin) {
    if (spin >= cap) {
      note_giveup();
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return v;
}

// Publish a counter after this wave's LDS writes.  The LDS unit performs one
// wave's operations in issue order, so the counter can never become
// visible before the data written ahead of it; only the compiler has to be
// kept from reordering, and no wait for completion is needed.
__device__ __forceinline__ void lds_publish(unsigned* p, unsigned v) {
  stress_delay(2);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The hand-off between consecutive workgroups of one pair ("segments") is
// done by one extra wave per workgroup, so the band waves never wait on
// global memory: it copies the new columns of the previous segment's bottom
// row from global memory into ring_in (the top ring of band 0), and what the
// last band wrote into ring_out to global memory.  Rows are accessed with
// relaxed agent-scope atomics (device-coherent loads and stores that bypass
// the per-XCD caches), so no cache write-back or invalidation is needed.
// The reader learns which columns are there in one of two ways:
//  - self-validating rows (valid_in / valid_out, whole rows only): the row
//    starts filled with kHEmpty, a signalling-NaN pattern that no
//    arithmetic produces (computed NaNs are quiet); the writer only stores
//    the values, and the reader polls the values themselves, takes the run
//    of columns no longer kHEmpty and writes kHEmpty back behind it, so the
//    row is ready for the next launch.  Values and markers are single
//    8-byte atomic accesses, so a value is never seen torn;
//  - counts: the writer waits for its stores (vmcnt(0)) and then publishes
//    the column count, which the reader polls before loading.
// A segment waits only on a smaller ticket, which is running, so the loop
// ends; the poll cap (per wait) guarantees the wave exits regardless.
//
// Global rows are either whole (hcols = 0: column c at H[c]) or rings of
// hcols columns (a power of two; column c at H[c % hcols]), which use
// counts.  With rings the consumer also publishes how many columns it has
// fetched (fetch_out) and the producer does not overwrite a slot before its
// consumer has fetched the column in it (fetch_back); that wait points at a
// larger ticket, so ring mode is only used where a pair's segments all fit
// on the GPU at once and tickets run pair by pair.
struct GlobalRow {
  unsigned hcols;             // 0: whole rows
  const unsigned* fetch_back; // consumer's fetched count (output side, ring mode)
  unsigned* fetch_out;        // own fetched count (input side, ring mode)
  bool valid_in = false;      // whole input row carries its own validity
  bool valid_out = false;     // whole output row carries its own validity
};

__device__ __forceinline__ void segment_io_wave(
    bool do_in, bool do_out, const unsigned* prog_in, unsigned* prog_out,
    const double* Hin, double* Hout, double* ring_in, unsigned* wr_in,
    const unsigned* rd_in, const double* ring_out, const unsigned* wr_out,
    unsigned* rd_out, unsigned M, int lane, GlobalRow gr = GlobalRow{0u, nullptr, nullptr}) {
  const unsigned hmask = gr.hcols ? gr.hcols - 1 : 0xffffffffu;
  unsigned fetched = 0, known_in = 0, pub = 0, known_back = 0;
  // Only a validated input row (always a workspace row) is written back.
  uint64_t* const hin_bits = reinterpret_cast<uint64_t*>(const_cast<double*>(Hin));
  // `idle` counts the polls since data last moved: the cap bounds each wait,
  // not the wave's lifetime (a long row moves data many times).
  const uint32_t cap = glob_cap();
  for (uint32_t idle = 0;;) {
    const bool in_left = do_in && fetched < M;
    const bool out_left = do_out && pub < M;
    if (!in_left && !out_left) break;
    if (idle >= cap) {
      note_giveup();
      break;
    }
    stress_delay(3);
    bool moved = false;
    if (in_left && gr.valid_in) {
      const unsigned room =
          __hip_atomic_load(rd_in, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + kRingC;
      unsigned lim = fetched + 64 < M ? fetched + 64 : M;
      lim = lim < room ? lim : room;
      const unsigned c = fetched + lane;
      uint64_t bits = kHEmpty;
      if (c < lim) bits = __hip_atomic_load(hin_bits + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t okm = __ballot(c < lim && bits != kHEmpty);
      const unsigned n = ~okm == 0 ? 64u : (unsigned)__builtin_ctzll(~okm);
      if (n > 0) {
        if ((unsigned)lane < n) {
          ring_in[c & (kRingC - 1)] = __builtin_bit_cast(double, bits);
          __hip_atomic_store(hin_bits + c, kHEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) lds_publish(wr_in, fetched + n);
        fetched += n;
        moved = true;
      }
    } else if (in_left) {
      if (known_in <= fetched)
        known_in = __hip_atomic_load(prog_in, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned room =
          __hip_atomic_load(rd_in, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + kRingC;
      const unsigned lim = known_in < room ? known_in : room;
      if (lim > fetched) {
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        for (unsigned c = fetched + lane; c < lim; c += 64)
          ring_in[c & (kRingC - 1)] =
              __hip_atomic_load(Hin + (c & hmask), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) lds_publish(wr_in, lim);
        if (gr.fetch_out && lane == 0)   // the loads above have returned
          __hip_atomic_store(gr.fetch_out, lim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        fetched = lim;
        moved = true;
      }
    }
    if (out_left) {
      unsigned avail = lds_wait_ge(wr_out, 0);
      if (gr.hcols) {
        if (avail > known_back + gr.hcols)
          known_back = __hip_atomic_load(gr.fetch_back, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        if (avail > known_back + gr.hcols) avail = known_back + gr.hcols;
      }
      if (avail > pub) {
        for (unsigned c = pub + lane; c < avail; c += 64)
          __hip_atomic_store(Hout + (c & hmask), ring_out[c & (kRingC - 1)], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) lds_publish(rd_out, avail);
        if (!gr.valid_out) {
          stress_delay(4);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_s_waitcnt(0);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (lane == 0)
            __hip_atomic_store(prog_out, avail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        pub = avail;
        moved = true;
      }
    }
    if (moved) {
      idle = 0;
    } else {
      __builtin_amdgcn_s_sleep(2);
      ++idle;
    }
  }
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

// The fused kernels' view: R holds original rows xrow0 .. of each pair in
// nbands bands, and the sweep rows of a launch may start anywhere.  The
// forward sweep's rows past the grid stay in the launch's last band; the
// reverse sweep's rows past the grid only load (their values are never
// used) and read row xrow0 + lane instead.
__device__ __forceinline__ LaneCursor lane_cursor_rows(bool rev, int64_t b, int64_t i,
                                                       int lane, int64_t N, int64_t M,
                                                       int nbands, int64_t S, int64_t xrow0) {
  LaneCursor c;
  if (!rev) {
    const int64_t r = i - xrow0;
    const int64_t l = r & 63;
    // cell (r, t - lane) is at step t - lane + l + off
    c.base = ((b * nbands + (r >> 6)) * S + (kSkewOff + l - lane)) * 64 + l;
    c.dir = 64;
  } else {
    const int64_t r = i < N ? N - 1 - i - xrow0 : lane;
    const int64_t l = r & 63;
    c.base = ((b * nbands + (r >> 6)) * S + (M - 1 + lane + l + kSkewOff)) * 64 + l;
    c.dir = -64;
  }
  return c;
}

}  // namespace sdtw

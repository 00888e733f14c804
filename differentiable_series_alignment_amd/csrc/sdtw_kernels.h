// Launch wrappers and the private data layout of the gfx950 Soft-DTW kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdtw {

// ---------------------------------------------------------------------------
// Band-step layout of the B x N x M cell arrays kept by the dynamic programme
// (distances / alignment matrix in fp32, forward state in fp64).
//
// Rows are grouped in bands of 64 (the last one padded); inside a band the
// cell (r, c) with lane l = r % 64 lives at step s = c + l + kSkewOff:
//     index(b, r, c) = ((b * nbands + r / 64) * S + (c + l + kSkewOff)) * 64 + l
// so the 64 cells one wavefront step touches (lane l at column t - l) are 64
// consecutive elements.  The reverse sweep, whose lanes walk columns from the
// right, reads the same steps with its lanes in reverse order.
//
// S is the distance between consecutive bands.  The sweeps store at every
// step they run, columns outside the grid included, so no such store may
// land on a cell of another band.  The cells at lane position l (the index
// mod 64) are one row's, at steps kSkewOff + l .. kSkewOff + l + M - 1 of
// their band, and a store at position l can only meet those.  A sweep lane
// working on the row at position l touches steps kSkewOff + [0, T) of the
// row's band (forward) or kSkewOff + l + j + M - 1 - [0, T) (reverse; j <=
// 63 is its lane in the reverse band), T = sweep_steps(M) >= M + 63.  With
// S = T (band_stride) both ranges lie after the previous band's last cell
// at that position (step kSkewOff + l + M - 1 - S) and before the next
// band's first (kSkewOff + l + S), for any N.  The fused kernels' R array
// uses the same stride: only their forward sweep stores into it, with the
// forward lanes' steps (a range launch's storage rows start at its first
// sweep row), and their reverse sweep only loads.  Kernels other than the
// sweeps store only cells.  An array holds band_array_elems(G, S, M)
// elements for G bands: the last band's frame extends over skew_steps(M)
// steps, room for every sweep access and for readers that clamp their steps
// below that.
// ---------------------------------------------------------------------------
constexpr int64_t kSkewOff = 80;

__host__ __device__ inline int64_t skew_steps(int64_t M) {
  return ((M + 2 * kSkewOff + 46 + 15) / 16) * 16;   // >= M + 206
}
__host__ __device__ inline int64_t skew_index(int64_t b, int64_t r, int64_t c,
                                              int64_t nbands, int64_t S) {
  const int64_t l = r & 63;
  return (((b * nbands + (r >> 6)) * S) + (c + l + kSkewOff)) * 64 + l;
}
// Steps a sweep runs per band: columns 0..M-1 for lanes 0..63, in chunks of 16.
__host__ __device__ inline int64_t sweep_steps(int64_t M) {
  return ((M + 63 + 15) / 16) * 16;
}
__host__ __device__ inline int64_t band_stride(int64_t M) { return sweep_steps(M); }
__host__ __device__ inline int64_t band_array_elems(int64_t G, int64_t S, int64_t M) {
  return ((G - 1) * S + skew_steps(M)) * 64;
}

// Marker of a hand-off entry not written yet: a signalling-NaN pattern,
// which no arithmetic produces (computed NaNs are quiet).
constexpr uint64_t kHEmpty = 0xFFF05D7C0DE0A11FULL;

// Arguments of the wavefront dynamic-programme kernels.  The forward sweep
// walks the grid from (0,0) to (N-1,M-1); the reverse sweep walks it from
// (N-1,M-1) back to (0,0), i.e. the forward recurrence on both sequences
// reversed.  All state is kept in base-2 units, X = R * log2(e) / gamma.
struct DPArgs {
  float* dsk;           // band-step distances (unfused)
  const float* x;       // [B,N,D] (fused)
  const float* y;       // [B,M,D] (fused)
  double* R;            // band-step forward state X
  double* R2;           // band-step reverse soft-minimum parts T' (unfused)
  double* H;            // bottom rows handed between segments
  int hvalid;           // whole H rows carry their own validity (start as
                        // kHEmpty, which every launch leaves behind)
  unsigned* ctrl;       // ticket, finished count, per-segment progress
  double* loss64;       // [B] X[N-1,M-1] (forward writes, reverse reads)
  float* loss;          // [B] loss in natural units (forward)
  const float* gl;      // [B] upstream gradients (fused reverse)
  float* gx;            // [B,N,D] (fused reverse; written)
  float* gy;            // [B,M,D] (fused reverse; accumulated, zeroed first)
  float* align;         // [B,N,M] optional E output (fused reverse)
  int64_t N, M, D, S;
  int B, nbands, nseg;
  double k2;            // log2(e) / gamma
  double g_ln2;         // gamma * ln(2) = 1 / k2
  // Fused kernels on a range of rows (checkpointed training).  The launch's
  // band k covers sweep rows row0 + 64k .. row0 + 64k + 63 (nseg bands);
  // R holds original rows xrow0 .. xrow0 + 64*nbands - 1.  When set, top_row
  // (row stride top_ld) is the complete row above the first band and bot_row
  // receives the last band's bottom row; full_word holds M and sink_word
  // takes the unused progress count.  All zero for whole-grid launches.
  int64_t row0, xrow0, top_ld;
  const double* top_row;
  double* bot_row;
  const unsigned* full_word;
  unsigned* sink_word;
  // Checkpoint rows written by the forward: original row r with
  // (N-1-r) = ck_span*(h+1), h < nck, goes to ckpt[(b*nck + h)*(M+2*kCkPad) + kCkPad + c].
  double* ckpt;
  int64_t ck_span;
  int nck;
  // Error word of the workspace (a wait gave up) and the test hook that
  // replaces the wait caps (0: built-in caps; sdtw_debug_wait_limit).
  unsigned* err;
  unsigned wait_cap;
  // Unfused sweeps of one launch: kSweepsBoth (forward and reverse at once,
  // the reverse keeping T' in R2), kSweepForward, or kSweepReverseE (the
  // reverse after a completed forward: it reads X from R and writes E over
  // the distances, then sets *eflag; a launch that finds *eflag set does
  // nothing, so E is formed once per forward).
  int sweeps;
  unsigned* eflag;
};
constexpr int kSweepsBoth = 0, kSweepForward = 1, kSweepReverseE = 2;
// Padding on each side of a stored checkpoint row (columns the band wave
// touches outside 0..M-1 land there).
constexpr int64_t kCkPad = 80;

// Bands (64 rows each) per workgroup of the DP kernels.
constexpr int kBandsPerWG = 4;
// Largest feature dimension the fused kernels handle (x rows of a band and the
// next distance block's y operand stay on chip).
constexpr int64_t kFusedMaxD = 256;
// Bands per workgroup of the fused kernels for this D (0: unsupported D).
int fused_bands_per_wg(int64_t D);

// Scope around one kernel launch: when launch timing is on, HIP events on
// `s` bracket the launch (see sdtw_timing).
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t s);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  hipStream_t stream_;
  long index_;
  hipEvent_t end_ = nullptr;
};

// While one exists on a host thread, launches on that thread are not timed
// (the allocation-free entry point creates no events).
class NoTimingScope {
 public:
  NoTimingScope();
  ~NoTimingScope();
  NoTimingScope(const NoTimingScope&) = delete;
  NoTimingScope& operator=(const NoTimingScope&) = delete;
};

// Body of sdtw_forward (include/sdtw.h), also behind sdtw_forward_static.
int forward_impl(const float* x, const float* y, int64_t B, int64_t N, int64_t M, int64_t D,
                 float gamma, int mode, void* workspace, size_t workspace_bytes, float* loss,
                 void* stream);

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s);
hipError_t launch_dist(const float* x, const float* y, float* dist, int64_t B,
                       int64_t N, int64_t M, int64_t D, hipStream_t stream);
// Band-step distances; also clears `nzero` words at `zero` (the step's
// control words) and sets `nempty` hand-off entries at `empty` to kHEmpty
// for the kernels that follow on the stream.
hipError_t launch_dist_skew(const float* x, const float* y, float* dsk, int64_t B,
                            int64_t N, int64_t M, int64_t D, int64_t S, unsigned* zero,
                            int64_t nzero, double* empty, int64_t nempty, hipStream_t stream);
// The same clearing alone.
hipError_t launch_clear(unsigned* zero, int64_t nzero, double* empty, int64_t nempty,
                        hipStream_t s);
hipError_t launch_unskew(const float* esk, float* out, int64_t B, int64_t N,
                         int64_t M, int64_t S, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
// Unfused: the sweeps of a.sweeps for every pair in one launch: both (X into
// R, T' into R2), the forward alone (X into R), or the reverse alone forming
// E over the distances (see DPArgs::sweeps).
hipError_t launch_dp_both(const DPArgs& a, hipStream_t s);
// Fused: one sweep per launch (the reverse one with the chain rule inside).
hipError_t launch_dp_fused(const DPArgs& a, bool reverse, hipStream_t s);
// Loss only: the fused forward sweep without stored state; hand-off rows are
// global rings of `hcols` columns (0: whole rows).  With a.ckpt set it also
// writes the checkpoint rows.
constexpr unsigned kHRing = 512;
hipError_t launch_infer(const DPArgs& a, unsigned hcols, hipStream_t s);
// Fused sweep over a range of rows (a.row0, a.nseg bands, see DPArgs): the
// forward one stores X of the range into R, the reverse one reads it.
hipError_t launch_fused_range(const DPArgs& a, bool reverse, hipStream_t s);
hipError_t launch_fill_u32(unsigned* p, int64_t n, unsigned v, hipStream_t s);
// Chain rule of the unfused backward.  The row pass forms E = 2^(Xnm-X-T')
// from R and R2 into `esk` (the distance array, no longer needed) and, if
// gx is given, writes dx; the column pass reads E from `esk` and writes dy.
// With D <= 64 and E not wanted afterwards (keep_e false) the row pass
// writes the bands' shares of dy into `esk` instead (chain_share_floats()
// floats, which `esk` must hold) and a short pass adds them up.  e_ready: E
// is already in `esk` (formed by the reverse sweep); every pass reads it and
// R, R2 are not used.  The arrays use the unfused band-step layout (band
// stride S = M).
// Small problems split each sum over several workgroups: `part` holds
// chain_part_floats() floats of partial sums and the counters (B*nbands for
// the rows, B*ceil(M/64) for the columns) start at zero and are left at zero.
int chain_splits_rows(int64_t B, int64_t N, int64_t M, int64_t D);
int chain_splits_cols(int64_t B, int64_t N, int64_t M);
size_t chain_part_floats(int64_t B, int64_t N, int64_t M, int64_t D);
size_t chain_share_floats(int64_t B, int64_t N, int64_t M, int64_t D);
hipError_t launch_chain(float* esk, const double* R, const double* R2,
                        const double* loss64, const float* x, const float* y,
                        const float* gl, float* gx, float* gy, int64_t B, int64_t N,
                        int64_t M, int64_t D, int64_t S, float* part, unsigned* cnt_rows,
                        unsigned* cnt_cols, bool keep_e, bool e_ready, hipStream_t s);

}  // namespace sdtw

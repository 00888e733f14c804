// Device helpers shared by the gfx950 Soft-DTW kernels (wave64 CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdtw {

typedef double v4d __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr double kInf = __builtin_inf();
constexpr double kLog2e = 1.4426950408889634073599246810019;
constexpr double kLn2 = 0.69314718055994530941723212145818;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Whole-wave shift towards higher lanes: lane l receives v from lane l-1;
// lane 0 receives `fill` (DPP wave_shr:1 with the bound-control bit clear
// keeps the destination's old value where the source lane does not exist).
__device__ __forceinline__ double wave_shr1(double v, double fill) {
  int lo = __double2loint(v), hi = __double2hiint(v);
  int flo = __double2loint(fill), fhi = __double2hiint(fill);
  int rlo = __builtin_amdgcn_update_dpp(flo, lo, 0x138, 0xF, 0xF, false);
  int rhi = __builtin_amdgcn_update_dpp(fhi, hi, 0x138, 0xF, 0xF, false);
  return __hiloint2double(rhi, rlo);
}

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// Stand-in for +inf in the DP state: far above any reachable state value
// (the state stays finite, so no inf - inf can ever produce a NaN) yet small
// enough that sums of a few hundred of them stay finite.
constexpr double kBig = 1e290;

// v_min_f64 / v_max_f64 on values known to be non-NaN (the generic fmin and
// fmax would first quiet possible signalling NaNs, which costs two extra
// instructions on the dependency chain of every step).
__device__ __forceinline__ double min_nonan(double a, double b) {
  double r;
  asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ double max_nonan(double a, double b) {
  double r;
  asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Soft-minimum part of one cell of the recurrence in base-2 units
// X = R * log2(e) / g:
//   X = d + T,  T = m - log2(2^(m-a) + 2^(m-b) + 2^(m-c)),  m = min(a, b, c),
// which is R = D + softmin_g(...) scaled by log2(e)/g.  The
// term of the minimum is exactly 1, so only the other two are
// exponentiated: with m1 = min(a,c), p = max(a,c), m = min(m1,b),
// q = max(m1,b), the multiset {a,b,c} is {m,p,q}.  State and differences
// are fp64; the exponentials and the logarithm are the fp32 hardware
// instructions applied to the (small, non-positive) fp64 differences.
//
// softmin2_cell returns the whole state X = (m + d) - log2(...) of a cell with
// scaled distance d, and sets t = T = m - log2(...): m + d is formed while
// the exponentials and the logarithm are in flight, so the distance costs no
// step on the dependency chain from one cell to the next.
__device__ __forceinline__ double softmin2_cell(double a, double b, double c, double d,
                                                double& t) {
  const double m1 = min_nonan(a, c);
  const double p = max_nonan(a, c);
  const double m = min_nonan(m1, b);
  const double q = max_nonan(m1, b);
  const double md = m + d;
  const float ep = hw_exp2((float)(m - p));
  const float eq = hw_exp2((float)(m - q));
  const double lg = (double)hw_log2((1.0f + ep) + eq);
  const double x = md - lg;
  t = m - lg;
  return x;
}

// Alignment-matrix entry from the two sweeps: with X the forward state of
// the cell, T' the soft-minimum part of the reverse state (the reverse
// state without the cell's own distance) and Xnm the final forward state,
//   log2 E = Xnm + d - X - X' = Xnm - X - T'.
__device__ __forceinline__ float align_entry(double xnm, double x, double tr) {
  return hw_exp2((float)((xnm - x) - tr));
}

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

}  // namespace sdtw

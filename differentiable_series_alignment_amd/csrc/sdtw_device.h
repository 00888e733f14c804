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

// One soft-min step of the recurrence in fp64 state with fp32
// transcendentals:  softmin_g(a,b,c) = m - g*ln(sum_k exp(-(a_k - m)/g)),
// m = min(a,b,c).  `k2` = log2(e)/g, `g_ln2` = g*ln(2); returns d + softmin.
// Infinite inputs contribute exp2(-inf) = 0; the result is garbage only when
// all three are +inf, which callers mask.
__device__ __forceinline__ double softmin_cell(double a, double b, double c,
                                               double d, double k2,
                                               double g_ln2) {
  double m = fmin(fmin(a, c), b);
  float ea = hw_exp2((float)((m - a) * k2));
  float eb = hw_exp2((float)((m - b) * k2));
  float ec = hw_exp2((float)((m - c) * k2));
  float s = (ea + ec) + eb;
  return fma(-g_ln2, (double)hw_log2(s), m + d);
}

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

}  // namespace sdtw

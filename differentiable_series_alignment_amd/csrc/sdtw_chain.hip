// Chain rule of Soft-DTW through the squared Euclidean distance (gfx950).
//
// With E = dloss/dDist (the alignment matrix) and Dist = ||x_i - y_j||^2:
//   dx[b,i,:] = 2 gl[b] (rowsum_i(E) x_i - sum_j E[i,j] y_j),
//   dy[b,j,:] = 2 gl[b] (colsum_j(E) y_j - sum_i E[i,j] x_i),
// i.e. two batched contractions E.Y and E^T.X (README "SoftDTW-CUDA (PyTorch +
// Numba)", "Usage": gradients of loss_fn(x, y).mean() reach x and y).
//
// E arrives in the band-step layout of the dynamic programme (see
// sdtw_kernels.h).  A workgroup stages a window of band steps in an LDS ring
// (coalesced: one step is 64 consecutive floats) and feeds
// v_mfma_f32_32x32x2_f32 from it.  Operand lanes: A[r][k] in lane r + 32k,
// B[k][c] in lane c + 32k; accumulator element (8*(e/4) + 4*(l/32) + e%4,
// l%32) in lane l, register e.  Ring rows are padded to 65 floats so both
// access patterns below hit distinct LDS banks.
#include "sdtw_device.h"
#include "sdtw_kernels.h"

namespace sdtw {

constexpr int kRingSteps = 128;
constexpr int kRingPitch = 65;
// Rows past the ring's end that mirror its first rows, so a run of up to
// kRingPad + 1 consecutive steps starting anywhere in the ring can be read
// at one base address plus constant offsets (no wrap-around per read).
constexpr int kRingPad = 32;
constexpr int kRingFloats = (kRingSteps + kRingPad) * kRingPitch;

// Row pitch (floats) of the bands' dy shares: D values and the column sum,
// rounded up to whole 16-byte words.
__host__ __device__ inline int64_t gy_pitch(int64_t D) { return (D + 4) & ~int64_t(3); }

// Copy band steps [s0, s0 + 32) (relative to the band's first column step)
// between global memory, registers and the LDS ring; 256 threads x 8 floats.
struct Stage32 {
  float v[8];
  __device__ __forceinline__ void load(const float* bandp, int64_t s0, int64_t smax) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = (int)threadIdx.x * 4 + 1024 * k;
      int64_t st = s0 + e / 64;
      st = st < smax ? st : smax - 1;
      const v4f q = *reinterpret_cast<const v4f*>(bandp + st * 64 + (e & 63));
      v[4 * k + 0] = q[0];
      v[4 * k + 1] = q[1];
      v[4 * k + 2] = q[2];
      v[4 * k + 3] = q[3];
    }
  }
  template <bool MIRROR = true>
  __device__ __forceinline__ void store(float* ring, int64_t s0) const {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = (int)threadIdx.x * 4 + 1024 * k;
      const int slot = (int)((s0 + e / 64) & (kRingSteps - 1));
#pragma unroll
      for (int q = 0; q < 4; ++q) ring[slot * kRingPitch + (e & 63) + q] = v[4 * k + q];
      if (MIRROR && slot < kRingPad) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ring[(slot + kRingSteps) * kRingPitch + (e & 63) + q] = v[4 * k + q];
      }
    }
  }
};

// The same 32-step window, formed from the two sweeps' states instead:
// E = 2^(Xnm - X - T') for each cell, written both to the LDS ring and to
// the band-step E array (the distance array, no longer needed) for the
// column pass and the optional alignment output.  Cells outside the grid
// (rows from rows_left on, columns outside 0..M-1) go to the ring as 0, so
// the products and sums over the ring need no masks; the E array receives
// only the grid's columns (a window's steps past a band's cells reach the
// next band's cells).
typedef double v2d __attribute__((ext_vector_type(2)));
struct StageXT {
  double xv[8], tv[8];
  int64_t off[2];
  __device__ __forceinline__ void load(const double* xbp, const double* tbp, int64_t s0,
                                       int64_t smax) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = (int)threadIdx.x * 4 + 1024 * k;
      int64_t st = s0 + e / 64;
      st = st < smax ? st : smax - 1;
      off[k] = st * 64 + (e & 63);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v2d a = *reinterpret_cast<const v2d*>(xbp + off[k] + 2 * h);
        const v2d c = *reinterpret_cast<const v2d*>(tbp + off[k] + 2 * h);
        xv[4 * k + 2 * h] = a[0];
        xv[4 * k + 2 * h + 1] = a[1];
        tv[4 * k + 2 * h] = c[0];
        tv[4 * k + 2 * h + 1] = c[1];
      }
    }
  }
  template <bool EOUT = true>
  __device__ __forceinline__ void store(float* ring, float* ebp, int64_t s0, double xnm,
                                        int rows_left, int64_t M) const {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = (int)threadIdx.x * 4 + 1024 * k;
      const int slot = (int)((s0 + e / 64) & (kRingSteps - 1));
      const int64_t col0 = s0 + e / 64 - (e & 63);   // column of lane (e & 63)
      v4f q;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = col0 - j;
        const bool ok = (e & 63) + j < rows_left && c >= 0 && c < M;
        q[j] = ok ? align_entry(xnm, xv[4 * k + j], tv[4 * k + j]) : 0.f;
        ring[slot * kRingPitch + (e & 63) + j] = q[j];
      }
      if (slot < kRingPad) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ring[(slot + kRingSteps) * kRingPitch + (e & 63) + j] = q[j];
      }
      if (EOUT) {
        // Columns col0 - 3 .. col0 of the four lanes; whole when all are in
        // the grid (the steps inside a band's ramps are stored word by word).
        if (col0 - 3 >= 0 && col0 < M) {
          __builtin_nontemporal_store(q, reinterpret_cast<v4f*>(ebp + off[k]));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (col0 - j >= 0 && col0 - j < M) ebp[off[k] + j] = q[j];
        }
      }
    }
  }
};

// Work item of a workgroup in a 1-D grid of 8 * ceil(W / 8) workgroups over
// W = n0 * n1 * n2 items (n0 fastest).  The GPU deals consecutive workgroups
// to its 8 XCDs in turn, so workgroup g takes item (g % 8) * ceil(W / 8) +
// g / 8: each XCD gets a contiguous run of items, and the items of one pair
// (consecutive in n0) share that XCD's L2.  Returns false past the last item.
struct WorkItem {
  int64_t i0, i1, i2;
};
__device__ __forceinline__ bool xcd_item(int64_t n0, int64_t n1, int64_t n2, WorkItem* it) {
  const int64_t per = (n0 * n1 * n2 + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= n0 * n1 * n2) return false;
  it->i0 = w % n0;
  it->i1 = (w / n0) % n1;
  it->i2 = w / (n0 * n1);
  return true;
}
__host__ inline unsigned xcd_grid(int64_t n0, int64_t n1, int64_t n2) {
  return (unsigned)(8 * ((n0 * n1 * n2 + 7) / 8));
}

// Split sums.  When the columns (dx) or the bands (dy) of one workgroup's sum
// are spread over `nsplit` workgroups, each writes its partial (the NTW
// accumulator tiles and the row or column sum, per thread) to `part`
// ([nsplit][16*NTW+1][256] floats for its group), and the last workgroup to
// arrive adds the partials in split order, so the result does not depend on
// the order of arrival.  Returns true in that last workgroup, which then
// holds the full sums and clears the group's counter for the next launch.
template <int NTW>
__device__ __forceinline__ bool split_reduce(v16f (&acc)[NTW], float& sum, float* part,
                                             unsigned* cnt, int p, int nsplit) {
  constexpr int K = 16 * NTW + 1;
  __shared__ unsigned s_last;
  const int tid = (int)threadIdx.x;
  // Partials go out as device-coherent stores (they bypass the per-XCD
  // caches); each thread waits for its own, the barrier makes that all of
  // them, and only then is the arrival counted.  The last workgroup reads
  // them back with device-coherent loads.  No cache write-back or
  // invalidation is needed for either side.
  float* mine = part + (int64_t)p * K * 256;
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      __hip_atomic_store(mine + (t * 16 + e) * 256 + tid, acc[t][e], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(mine + 16 * NTW * 256 + tid, sum, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(nsplit - 1);
  __syncthreads();
  if (!s_last) return false;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  sum = 0.f;
  for (int q = 0; q < nsplit; ++q) {
    const float* src = part + (int64_t)q * K * 256;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] += __hip_atomic_load(
          src + (t * 16 + e) * 256 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sum += __hip_atomic_load(src + 16 * NTW * 256 + tid, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// dx for one band (64 rows) of one pair, columns of D in [d0, d0 + 128).
// Wave w: row tile w & 1, d tiles (w >> 1) + 2t.  Column blocks of 32 need
// band steps [j0, j0 + 96); the next block's 32 new steps are fetched into
// registers while the current block computes, and its y rows once this
// block's products are issued (one register set for y instead of two:
// 4096x1000, D=128 627 us against 704; 32x512x512 61 against 64).  FORM: the window comes from
// the sweeps' states and E is formed (and stored) on the way; otherwise it
// is read from the stored E.  GX = false forms E only.  The band's column
// blocks are split over nsplit workgroups (split sums, above).
//
// GYP (D <= 64, FORM): E is not stored; instead each block also yields the
// band's shares of dy for its 32 columns: P[b][band][j][d] = -sum over the
// band's rows i of E[i,j] x_i[d] (d < D) and P[b][band][j][D] = sum of
// E[i,j], into `esk` viewed as [B][nbands][M][gy_pitch(D)] (k_chain_gy adds
// the bands up).  Wave w: d tile w >> 1, rows 32 (w & 1) .. +31; the two row
// halves meet in LDS.
template <int NTW, bool GX, bool FORM, bool GYP>
__global__ __launch_bounds__(256) void k_chain_rows(float* __restrict__ esk,
                                                    const double* __restrict__ R,
                                                    const double* __restrict__ R2,
                                                    const double* __restrict__ loss64,
                                                    const float* __restrict__ x,
                                                    const float* __restrict__ y,
                                                    const float* __restrict__ gl,
                                                    float* __restrict__ gx, int64_t N,
                                                    int64_t M, int64_t D, int64_t S,
                                                    int nbands, int64_t d0,
                                                    float* __restrict__ part,
                                                    unsigned* __restrict__ cnt,
                                                    int64_t nb_pairs, int nsplit) {
  __shared__ float ring[kRingFloats];
  WorkItem it;
  // The split parts of a band are consecutive items (same XCD, dispatched
  // together), so the window steps they both read come from one L2.
  if (!xcd_item(nsplit, nbands, nb_pairs, &it)) return;
  const int64_t b = it.i2, band = it.i1;
  const int p = (int)it.i0;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r = l & 31, h = l >> 5;
  const int rt = w & 1, dsel = w >> 1;
  const int lr = 32 * rt + r;
  const int64_t row = band * 64 + lr;
  const bool row_ok = row < N;
  const int rows_left = (int)(N - band * 64 < 64 ? N - band * 64 : 64);
  const int64_t boff = ((b * nbands + band) * S + kSkewOff) * 64;
  float* bandp = esk + boff;
  const double* xbp = R + boff;
  const double* tbp = R2 + boff;
  const double xnm = FORM ? loss64[b] : 0.0;
  const int64_t smax = skew_steps(M) - kSkewOff;   // reads stay in the array
  const float* yb = y + b * M * D;
  int64_t dcol[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int64_t dc = d0 + 32 * (dsel + 2 * t) + r;
    dcol[t] = dc < D ? dc : D - 1;
  }
  v16f acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  float rsum = 0.f;

  const int64_t nblk = (M + 31) / 32;
  const int64_t kb0 = p * nblk / nsplit, kb1 = (p + 1) * nblk / nsplit;
  Stage32 st;
  StageXT sx;
  for (int64_t s0 = kb0 * 32; s0 < kb0 * 32 + 96; s0 += 32) {
    if (FORM) {
      sx.load(xbp, tbp, s0, smax);
      sx.template store<!GYP>(ring, bandp, s0, xnm, rows_left, M);
    } else {
      st.load(bandp, s0, smax);
      st.store(ring, s0);
    }
  }
  float yv[16][NTW];
  auto load_y = [&](int64_t j0, float (&Y)[16][NTW]) {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      int64_t j = j0 + 2 * s + h;
      j = j < M ? j : M - 1;
#pragma unroll
      for (int t = 0; t < NTW; ++t) Y[s][t] = yb[j * D + dcol[t]];
    }
  };
  if (GX) load_y(kb0 * 32, yv);
  // GYP: this wave's x rows (B operand of E^T . X, fixed for the band) and
  // the LDS area where the second row half hands over its sums.
  const int gdt = w >> 1, grh = w & 1;
  const int64_t gd = 32 * gdt + r;                 // column of D
  float xg[16];
  __shared__ float gsum[GYP ? 2 * 17 * 64 : 1];
  if (GYP) {
    const float* xb = x + b * N * D;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      int64_t rr = band * 64 + 32 * grh + 2 * s + h;
      rr = rr < N ? rr : N - 1;
      xg[s] = gd < D ? xb[rr * D + gd] : 0.f;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int64_t kb = kb0; kb < kb1; ++kb) {
    const int64_t j0 = kb * 32;
    const bool more = kb + 1 < kb1;
    if (more) {
      if (FORM)
        sx.load(xbp, tbp, j0 + 96, smax);
      else
        st.load(bandp, j0 + 96, smax);
    }
    if (GX) {
      // E[row, j0 + 2s + h] for s = 0..15: ring rows base + 2s (the pad
      // mirrors the wrap), all read before the first product.
      const float* ea = ring + (int)((j0 + h + lr) & (kRingSteps - 1)) * kRingPitch + lr;
      float ev[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) ev[s] = ea[s * 2 * kRingPitch];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int64_t j = j0 + 2 * s + h;
        const float a = (FORM || (row_ok && j < M)) ? ev[s] : 0.f;   // FORM: masked
        rsum += a;
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, yv[s][t], acc[t], 0, 0, 0);
      }
      if (more) load_y(j0 + 32, yv);
    }
    v16f gacc;
    float gcs = 0.f;
    if (GYP) {
      // E^T . X over this wave's 32 rows: A[j][k] = E[row 32*grh + 2s + k,
      // column j0 + j] in lane j + 32k.
#pragma unroll
      for (int e = 0; e < 16; ++e) gacc[e] = 0.f;
      const int64_t j = j0 + r;
      const int lrow0 = 32 * grh + h;
      const float* eg = ring + (int)((j + lrow0) & (kRingSteps - 1)) * kRingPitch + lrow0;
      float ev[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) ev[s] = eg[s * (2 * kRingPitch + 2)];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const float a = ev[s];   // cells outside the grid were stored as 0
        gcs += a;
        gacc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, xg[s], gacc, 0, 0, 0);
      }
      gcs += __shfl_xor(gcs, 32, 64);          // column sums over this half
      if (grh == 1) {
#pragma unroll
        for (int e = 0; e < 16; ++e) gsum[(gdt * 17 + e) * 64 + l] = gacc[e];
        gsum[(gdt * 17 + 16) * 64 + l] = gcs;
      }
    }
    __syncthreads();
    if (GYP && grh == 0) {
      // P[j][d] = colsum_j y_j[d] - (E^T X)[j][d] for the band's 64 rows.
#pragma unroll
      for (int e = 0; e < 16; ++e) gacc[e] += gsum[(gdt * 17 + e) * 64 + l];
      gcs += gsum[(gdt * 17 + 16) * 64 + l];
      const int64_t D1 = gy_pitch(D);
      float* pb = esk + (b * nbands + band) * M * D1;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jr = 8 * (e >> 2) + 4 * h + (e & 3);   // accumulator row
        const int64_t jj = j0 + jr;
        if (jj < M && gd < D) pb[jj * D1 + gd] = -gacc[e];
      }
      if (gdt == 0 && h == 0 && j0 + r < M) pb[(j0 + r) * D1 + D] = gcs;
    }
    if (more) {
      if (FORM)
        sx.template store<!GYP>(ring, bandp, j0 + 96, xnm, rows_left, M);
      else
        st.store(ring, j0 + 96);

    }
    __syncthreads();
  }
  if (!GX) return;
  if (nsplit > 1 &&
      !split_reduce<NTW>(acc, rsum, part + (b * nbands + band) * (int64_t)nsplit * (16 * NTW + 1) * 256,
                         cnt + b * nbands + band, p, nsplit))
    return;

  rsum += __shfl_xor(rsum, 32, 64);
  float rs[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) rs[e] = __shfl(rsum, 8 * (e >> 2) + 4 * h + (e & 3), 64);
  const float g2 = 2.f * gl[b];
  const float* xb = x + b * N * D;
  float* ob = gx + b * N * D;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int64_t dc = d0 + 32 * (dsel + 2 * t) + r;
    if (dc >= D || dc >= d0 + 128) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t orow = band * 64 + 32 * rt + 8 * (e >> 2) + 4 * h + (e & 3);
      if (orow < N) ob[orow * D + dc] = g2 * (rs[e] * xb[orow * D + dc] - acc[t][e]);
    }
  }
}

// dy for 64 columns of one pair, columns of D in [d0, d0 + 128), summing over
// every band.  Wave w: column tile w & 1, d tiles (w >> 1) + 2t.  The band's
// window of steps [j0, j0 + 128) is fetched into registers one band ahead;
// the next band's x rows are fetched once this band's products are issued
// (a second register set for them would leave one wave per SIMD: 280
// VGPRs against 228, and 4096x1000, D=128 takes 584 us against 442).
// The bands are split over nsplit workgroups (split sums, above).
template <int NTW>
__global__ __launch_bounds__(256) void k_chain_cols(const float* __restrict__ esk,
                                                    const float* __restrict__ x,
                                                    const float* __restrict__ y,
                                                    const float* __restrict__ gl,
                                                    float* __restrict__ gy, int64_t N,
                                                    int64_t M, int64_t D, int64_t S,
                                                    int nbands, int64_t d0,
                                                    float* __restrict__ part,
                                                    unsigned* __restrict__ cnt,
                                                    int64_t nb_pairs, int nsplit) {
  __shared__ float ring[kRingSteps * kRingPitch];
  const int64_t ncb = (M + 63) / 64;
  WorkItem it;
  if (!xcd_item(nsplit, ncb, nb_pairs, &it)) return;
  const int64_t b = it.i2, cb = it.i1, j0 = cb * 64;
  const int p = (int)it.i0;
  const int64_t bb0 = (int64_t)p * nbands / nsplit, bb1 = (int64_t)(p + 1) * nbands / nsplit;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r = l & 31, h = l >> 5;
  const int ct = w & 1, dsel = w >> 1;
  const int jl = 32 * ct + r;
  const bool col_ok = j0 + jl < M;
  const int64_t smax = skew_steps(M) - kSkewOff;   // reads stay in the array
  const float* xb = x + b * N * D;
  int64_t dcol[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int64_t dc = d0 + 32 * (dsel + 2 * t) + r;
    dcol[t] = dc < D ? dc : D - 1;
  }
  v16f acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  float csum = 0.f;

  Stage32 win[4], nxt[4];
  float xv[32][NTW];
  auto load_win = [&](int64_t band, Stage32 (&Wn)[4]) {
    const float* bandp = esk + ((b * nbands + band) * S + kSkewOff) * 64;
#pragma unroll
    for (int k = 0; k < 4; ++k) Wn[k].load(bandp, j0 + 32 * k, smax);
  };
  auto load_x = [&](int64_t band, float (&X)[32][NTW]) {
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      int64_t rr = band * 64 + 2 * s + h;
      rr = rr < N ? rr : N - 1;
#pragma unroll
      for (int t = 0; t < NTW; ++t) X[s][t] = xb[rr * D + dcol[t]];
    }
  };
  load_win(bb0, win);
  load_x(bb0, xv);
  __builtin_amdgcn_s_waitcnt(0);

  for (int64_t band = bb0; band < bb1; ++band) {
#pragma unroll
    for (int k = 0; k < 4; ++k) win[k].template store<false>(ring, 32 * k);
    __syncthreads();
    const bool more = band + 1 < bb1;
    if (more) load_win(band + 1, nxt);
    // Steps jl + lr of rows lr = 2s + h (no wrap: jl + lr < 128), all read
    // before the first product.
    float ev[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) ev[s] = ring[(jl + 2 * s + h) * kRingPitch + 2 * s + h];
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int lr = 2 * s + h;
      const bool ok = col_ok && band * 64 + lr < N;
      const float a = ok ? ev[s] : 0.f;
      csum += a;
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, xv[s][t], acc[t], 0, 0, 0);
    }
    if (more) load_x(band + 1, xv);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int k = 0; k < 4; ++k) win[k] = nxt[k];
    }
  }

  if (nsplit > 1 &&
      !split_reduce<NTW>(acc, csum, part + (b * ncb + cb) * (int64_t)nsplit * (16 * NTW + 1) * 256,
                         cnt + b * ncb + cb, p, nsplit))
    return;

  csum += __shfl_xor(csum, 32, 64);
  float cs[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) cs[e] = __shfl(csum, 8 * (e >> 2) + 4 * h + (e & 3), 64);
  const float g2 = 2.f * gl[b];
  const float* yb = y + b * M * D;
  float* ob = gy + b * M * D;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int64_t dc = d0 + 32 * (dsel + 2 * t) + r;
    if (dc >= D || dc >= d0 + 128) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t oj = j0 + 32 * ct + 8 * (e >> 2) + 4 * h + (e & 3);
      if (oj < M) ob[oj * D + dc] = g2 * (cs[e] * yb[oj * D + dc] - acc[t][e]);
    }
  }
}

// dy[b,j,d] = 2 g_b (y[b,j,d] sum_k P[b][k][j][D] + sum_k P[b][k][j][d]),
// the bands k added in order (the shares the row pass wrote with GYP).  A
// thread takes four consecutive d of one row j (rows of gy_pitch(D) floats,
// so every share row starts on 16 bytes and is read as whole 16-byte
// words; the last word of a row holds the column sum).
__global__ __launch_bounds__(256) void k_chain_gy(const float* __restrict__ P,
                                                  const float* __restrict__ y,
                                                  const float* __restrict__ gl,
                                                  float* __restrict__ gy, int64_t B, int64_t M,
                                                  int64_t D, int nbands) {
  const int64_t D1 = gy_pitch(D), nq = (D + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= B * M * nq) return;
  const int64_t bj = i / nq, q = i - bj * nq;
  const int64_t b = bj / M, j = bj - b * M;
  const float* pp = P + (b * nbands * M + j) * D1;
  float cs = 0.f;
  v4f ex = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < nbands; ++k) {
    const float* row = pp + (int64_t)k * M * D1;
    cs += row[D];
    ex += *reinterpret_cast<const v4f*>(row + 4 * q);
  }
  const float g2 = 2.f * gl[b];
  const float* yr = y + bj * D;
  float* out = gy + bj * D;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t d = 4 * q + u;
    if (d < D) out[d] = g2 * (cs * yr[d] + ex[u]);
  }
}

// Whether the row pass makes the per-band shares of dy: D <= 64 (one d
// tile), and the shares of a band take no more floats than a band of the
// padded band-step layout (skew_steps(M) steps); beyond that (M > 3296) E
// is stored and read back by the column pass.
static bool chain_gy_path(int64_t M, int64_t D) {
  return D <= 64 && M * gy_pitch(D) <= skew_steps(M) * 64;
}

size_t chain_share_floats(int64_t B, int64_t N, int64_t M, int64_t D) {
  return chain_gy_path(M, D) ? (size_t)(B * ((N + 63) / 64) * M * gy_pitch(D)) : 0;
}

// Row-pass splits when it makes the dy shares.  Every part first loads a
// 96-step window, so short parts mostly load: the parts fill the GPU with
// one workgroup per CU keeping at least two column blocks each, or with two
// per CU keeping at least four, whichever splits more.
// Measured: 32x256x256 31 us with two parts per band against 34 with four;
// 10x100x100 18 us with two against 22 unsplit; 32x1024x1024 194 us
// unsplit against 213 with two; 32x512x512 the same with two to four.
static int chain_splits_rows_gy(int64_t B, int64_t N, int64_t M) {
  const int64_t nb = (N + 63) / 64, groups = B * nb, nblk = (M + 31) / 32;
  int64_t p1 = (256 + groups - 1) / groups, p2 = (512 + groups - 1) / groups;
  p1 = p1 < nblk / 2 ? p1 : nblk / 2;
  p2 = p2 < nblk / 4 ? p2 : nblk / 4;
  int64_t p = p1 > p2 ? p1 : p2;
  p = p < 1 ? 1 : (p > 8 ? 8 : p);
  return (int)p;
}

// Workgroups per band (dx) or per 64-column block (dy): a launch with fewer
// groups than the GPU has CUs splits each group's reduction range so that it
// fills them, keeping at least two column blocks (or bands) per workgroup.
// Larger launches do not split (a split gains nothing there and its partial
// sums would cost memory).  Where the dy shares can be made, the row pass
// splits as the share path does whether or not E is requested, so dx is
// summed in the same order either way.
constexpr int64_t kChainFill = 256;
int chain_splits_rows(int64_t B, int64_t N, int64_t M, int64_t D) {
  if (chain_gy_path(M, D)) return chain_splits_rows_gy(B, N, M);
  const int64_t groups = B * ((N + 63) / 64), nblk = (M + 31) / 32;
  int64_t p = (kChainFill + groups - 1) / groups;
  p = p < nblk / 2 ? p : nblk / 2;
  return (int)(p < 1 ? 1 : (p > 8 ? 8 : p));
}
int chain_splits_cols(int64_t B, int64_t N, int64_t M) {
  const int64_t groups = B * ((M + 63) / 64), nb = (N + 63) / 64;
  int64_t p = (kChainFill + groups - 1) / groups;
  p = p < nb / 2 ? p : nb / 2;
  return (int)(p < 1 ? 1 : (p > 8 ? 8 : p));
}
// Each split part holds 16 * NTW + 1 rows of 256 floats; NTW = 2 only where
// a D slice is wider than 64.
size_t chain_part_floats(int64_t B, int64_t N, int64_t M, int64_t D) {
  const int64_t pr = chain_splits_rows(B, N, M, D), pc = chain_splits_cols(B, N, M);
  const int64_t rows = pr > 1 ? B * ((N + 63) / 64) * pr : 0;
  const int64_t cols = pc > 1 ? B * ((M + 63) / 64) * pc : 0;
  const int64_t k = D > 64 ? 33 : 17;
  return (size_t)(rows > cols ? rows : cols) * k * 256;
}

template <int NTW, bool FORM, bool GYP = false>
static void launch_rows(int64_t B, unsigned nsplit, hipStream_t s, float* esk,
                        const double* R, const double* R2, const double* loss64,
                        const float* x, const float* y, const float* gl, float* gx, int64_t N,
                        int64_t M, int64_t D, int64_t S, int nb, int64_t d0, float* part,
                        unsigned* cnt) {
  const dim3 grid(xcd_grid(nb, B, nsplit));
  TimedLaunch timed_("chain_rows", s);
  if (gx)
    hipLaunchKernelGGL((k_chain_rows<NTW, true, FORM, GYP>), grid, dim3(256), 0, s, esk, R, R2,
                       loss64, x, y, gl, gx, N, M, D, S, nb, d0, part, cnt, B, (int)nsplit);
  else
    hipLaunchKernelGGL((k_chain_rows<1, false, FORM, GYP>), grid, dim3(256), 0, s, esk, R, R2,
                       loss64, x, y, gl, gx, N, M, D, S, nb, d0, part, cnt, B, (int)nsplit);
}

hipError_t launch_chain(float* esk, const double* R, const double* R2,
                        const double* loss64, const float* x, const float* y,
                        const float* gl, float* gx, float* gy, int64_t B, int64_t N,
                        int64_t M, int64_t D, int64_t S, float* part, unsigned* cnt_rows,
                        unsigned* cnt_cols, bool keep_e, bool e_ready, hipStream_t s) {
  const int nb = (int)((N + 63) / 64);
  const unsigned pr = (unsigned)chain_splits_rows(B, N, M, D);
  const unsigned pc = (unsigned)chain_splits_cols(B, N, M);
  if (gy && !keep_e && !e_ready && chain_gy_path(M, D)) {
    // One row pass makes dx and the bands' shares of dy (in place of E);
    // a short pass adds the shares up.
    launch_rows<1, true, true>(B, pr, s, esk, R, R2, loss64, x, y, gl, gx, N, M, D, S, nb, 0,
                               part, cnt_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    TimedLaunch timed_("chain_gy", s);
    hipLaunchKernelGGL(k_chain_gy, dim3((unsigned)((B * M * ((D + 3) / 4) + 255) / 256)), dim3(256), 0, s,
                       esk, y, gl, gy, B, M, D, nb);
    return hipGetLastError();
  }
  // Row pass(es): the first forms E; later D slices read it back.
  for (int64_t d0 = 0; d0 < D; d0 += 128) {
    if (d0 > 0 && !gx) break;
    const int64_t dw = D - d0 < 128 ? D - d0 : 128;
    const bool two = dw > 64;  // more than two 32-wide d tiles
    if (d0 == 0 && !e_ready) {
      if (two)
        launch_rows<2, true>(B, pr, s, esk, R, R2, loss64, x, y, gl, gx, N, M, D, S, nb, d0, part, cnt_rows);
      else
        launch_rows<1, true>(B, pr, s, esk, R, R2, loss64, x, y, gl, gx, N, M, D, S, nb, d0, part, cnt_rows);
    } else {
      if (two)
        launch_rows<2, false>(B, pr, s, esk, R, R2, loss64, x, y, gl, gx, N, M, D, S, nb, d0, part, cnt_rows);
      else
        launch_rows<1, false>(B, pr, s, esk, R, R2, loss64, x, y, gl, gx, N, M, D, S, nb, d0, part, cnt_rows);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!gy) return hipSuccess;
  for (int64_t d0 = 0; d0 < D; d0 += 128) {
    const int64_t dw = D - d0 < 128 ? D - d0 : 128;
    const dim3 grid(xcd_grid((M + 63) / 64, B, pc));
    TimedLaunch timed_("chain_cols", s);
    if (dw > 64)
      hipLaunchKernelGGL(k_chain_cols<2>, grid, dim3(256), 0, s, esk, x, y, gl, gy, N, M, D, S, nb, d0, part, cnt_cols, B, (int)pc);
    else
      hipLaunchKernelGGL(k_chain_cols<1>, grid, dim3(256), 0, s, esk, x, y, gl, gy, N, M, D, S, nb, d0, part, cnt_cols, B, (int)pc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sdtw

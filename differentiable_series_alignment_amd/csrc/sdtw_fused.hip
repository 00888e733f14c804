// Fused-distance wavefront kernels (gfx950): no B x N x M distance tensor.
//
// The README "SoftDTW-CUDA (PyTorch + Numba)" ("Fused Mode": no distance
// tensor; "Limitations": squared Euclidean only) and the review page
// "SoftDTW-CUDA-Torch" ("Proposed method": distances recomputed on the fly)
// describe a mode that never materialises Dist.  Here one workgroup owns one
// 64-row band of one pair, and its waves split the work so that the
// dependency chain of the sweep never waits on a matrix instruction:
//  - the band wave runs the recurrence (lane = row, as in the unfused
//    kernel) and reads each cell's distance from an LDS ring;
//  - distance helper waves compute the ring's 64 x 16 blocks ahead of it on
//    fp64 MFMA, from the band's x rows (resident in LDS) and the y rows of
//    the block, with the same operations in the same order as the distance
//    kernel, so fused and unfused distances are bit-identical;
//  - in the reverse sweep the band wave replaces each ring entry by its
//    alignment value E = 2^(Xnm - X - T') once the cell is done, and
//    chain-rule helper waves consume every completed 16-column block on
//    fp32 MFMA: dx of the band's rows (kept in registers; each helper owns a
//    slice of the columns of D) and dy of the block's columns (atomic adds:
//    the bands share columns);
//  - one wave hands the band's bottom row to the next band's workgroup and
//    receives the row above from the previous one (segment_io_wave).
// All coordination inside a workgroup goes through LDS counters.
#include <type_traits>

#include "sdtw_dp_common.h"

namespace sdtw {

// Distance/E ring columns per band (16 blocks of 16; see launch_fused_one).
constexpr int kFR = 256;
constexpr int kFPitch = 66;  // floats per ring column: 64 rows + 2 (LDS banks)
constexpr int kFwdHelpD = 3; // distance helpers, forward sweep (D <= 64)
constexpr int kFwdHelpDWide = 6; // distance helpers, forward sweep (D > 64)
constexpr int kRevHelpD = 2; // distance helpers, reverse sweep (3 for D <= 32, 64 < D <= 192)
constexpr int kRevHelpCMax = 4;
constexpr int kYB = 16;      // feature steps (of 4) per batch of y loads

__host__ __device__ constexpr int fused_pitch(int64_t D) { return (int)(((D + 3) / 4) * 4 + 4); }

// y rows staged for a chain-rule helper: blocks of 16 rows, DC columns of D
// each, rows padded by 2 floats (LDS banks).  Two blocks (the next one
// staged while the current one is in use) up to DC = 32; one for the
// 64-column helpers, whose workgroups (D > 128) could not otherwise hold the
// 256-column ring next to x rows of up to 256 features: 32 x 256^2, D=256,
// reverse sweep 306 -> 259 us with the deeper ring, no change at D = 192.
__host__ __device__ constexpr int chain_y_bufs(int DC) { return DC > 32 ? 1 : 2; }
__host__ __device__ constexpr int chain_y_floats(int DC) { return chain_y_bufs(DC) * 16 * (DC + 2); }

// Dynamic LDS of one workgroup: the band's x rows and the distance/E ring,
// plus (reverse sweep, HC chain-rule helpers of DC columns of D each) the
// helpers' staged y rows.
constexpr size_t fused_lds_bytes(int64_t D, int DC, int HC, int FR) {
  return (size_t)64 * fused_pitch(D) * 4 + (size_t)FR * kFPitch * 4 +
         (DC ? (size_t)HC * chain_y_floats(DC) * 4 : 0);
}

// One band per workgroup; 0 when D is beyond what the kernels hold on chip.
int fused_bands_per_wg(int64_t D) { return (D >= 1 && D <= kFusedMaxD) ? 1 : 0; }

struct FusedShared {
  double ring_in[kRingC + kCH];   // row above the band (from the previous band)
  double ring_out[kRingC + kCH];  // the band's bottom row (to the next band)
  unsigned wr_in, rd_in, wr_out, rd_out;
  unsigned d_ready;               // distance blocks published, in order
  unsigned dp_done;               // chunks completed by the band wave
  unsigned e_free[kRevHelpCMax];  // blocks released by each chain-rule helper
  unsigned x_done[kRevHelpCMax];  // dx partials handed over (helper pairs)
  unsigned ticket;
};

__device__ __forceinline__ unsigned umin_u(unsigned a, unsigned b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// Band wave.
// ---------------------------------------------------------------------------
template <bool REV, bool STORE, bool CKPT, bool SPLIT, int FR>
__device__ __forceinline__ void fused_band(const DPArgs& a, FusedShared& sh, float* dr, int b,
                                           int band, int lane) {
  const int64_t N = a.N, M = a.M, S = a.S;
  const int64_t r0 = a.row0 + (int64_t)band * 64;
  const int64_t i = r0 + lane;
  const int qcount = (int)(sweep_steps(M) / kCH);
  const bool top_ring = band > 0 || a.top_row != nullptr;
  const bool out_used = band + 1 < a.nseg || a.bot_row != nullptr;
  // With self-validating rows a band hands its bottom row straight to the
  // next band's row in global memory (no LDS ring, no copy by the hand-off
  // wave); the last band of a range launch still goes through the hand-off
  // wave to bot_row.  The hand-off wave makes the same choice.
  const bool direct_out = a.hvalid != 0 && band + 1 < a.nseg;
  double* const hout = direct_out ? a.H + ((int64_t)b * a.nseg + band) * M : nullptr;
  const unsigned Mu = (unsigned)M;
  const LaneCursor cu = lane_cursor_rows(REV, b, i, lane, N, M, a.nbands, S, a.xrow0);
  double* const rbase = (REV || STORE) ? a.R + cu.base : nullptr;
  const double k2 = a.k2;
  const double xnm = REV ? a.loss64[b] : 0.0;
  const int64_t lastrow = N - 1;
  const bool has_last = !REV && a.loss != nullptr && lastrow >= r0 && lastrow < r0 + 64;
  const int64_t tlast = M - 1 + (lastrow - r0);
  const int qlast = (int)(tlast / kCH), ulast = (int)(tlast % kCH);
  // Checkpoint row of this lane (forward, CKPT): stored for every step, its
  // columns outside 0..M-1 going to the row's padding.
  double* ckp = nullptr;
  bool band_ck = false;
  if (CKPT) {
    const int64_t back = N - 1 - i;
    const bool ck = i < N && back > 0 && back % a.ck_span == 0 && back / a.ck_span <= a.nck;
    if (ck)
      ckp = a.ckpt + ((int64_t)b * a.nck + (back / a.ck_span - 1)) * (M + 2 * kCkPad) + kCkPad -
            lane;
    band_ck = __ballot(ck) != 0;
  }
  float* alignp = (REV && a.align && i < N) ? a.align + ((int64_t)b * N + (N - 1 - i)) * M
                                            : nullptr;
  constexpr int dir = REV ? -64 : 64;

  double cur = kBig;
  double up = (r0 == 0 && lane == 0) ? 0.0 : kBig;
  unsigned seen_wr = 0, seen_rd = 0, seen_d = 0;

  // Reverse sweep: the forward state of the chunk's cells, requested one
  // chunk ahead into alternating register sets.
  double rnA[kCH], rnB[kCH];
  auto load_x = [&](int q, double (&R_)[kCH]) {
    const double* p0 = rbase + (int64_t)q * kCH * dir;
    const double* p8 = p0 + 8 * dir;
#pragma unroll
    for (int u = 0; u < kCH; ++u) R_[u] = (u < 8 ? p0 : p8)[(u & 7) * dir];
  };
  if (REV) load_x(0, rnA);

  auto chunk = [&](int q, const double (&rn)[kCH], double (&rn2)[kCH]) {
    const int t0 = q * kCH;
    double top[kCH];
    if (top_ring) {
      const unsigned need = umin_u((unsigned)t0 + kCH, Mu);
      if (seen_wr < need) seen_wr = lds_wait_ge(&sh.wr_in, need);
#pragma unroll
      for (int u = 0; u < kCH; ++u) top[u] = sh.ring_in[(t0 + u) & (kRingC - 1)];
    } else {
#pragma unroll
      for (int u = 0; u < kCH; ++u) top[u] = kBig;
    }
    if (REV) load_x(q + 1 < qcount ? q + 1 : q, rn2);
    // Distances of the chunk's cells: blocks 0..q must be in the ring.
    if (seen_d < (unsigned)q + 1) seen_d = lds_wait_ge(&sh.d_ready, (unsigned)q + 1);
    float dn[kCH];
#pragma unroll
    for (int u = 0; u < kCH; ++u) dn[u] = dr[((t0 + u - lane) & (FR - 1)) * kFPitch + lane];

    double bottom[kCH];
    double* sp = rbase + (int64_t)t0 * dir;
    double* sp8 = sp + 8 * dir;
    // MASK: the chunk holds cells of columns < 0 (only the first 64 steps
    // do); ALIGN: E also goes to the optional alignment output.  With SPLIT
    // both are fixed per chunk (four copies of the step loop), so most
    // chunks carry no per-step test for them: 3-5 % off the reverse sweep,
    // at the cost of ~40 more VGPRs, which only workgroups of up to eight
    // waves can afford (nine waves would spill).
    auto run_steps = [&](auto mask_c, auto align_c) {
      constexpr bool MASK = decltype(mask_c)::value;
      constexpr bool ALIGN = decltype(align_c)::value;
#pragma unroll
      for (int u = 0; u < kCH; ++u) {
        const int t = t0 + u;
        const bool boundary = MASK && t < lane;   // column < 0
        double d = (double)dn[u] * k2;
        if (MASK) d = boundary ? kBig : d;
        const double upn = wave_shr1(cur, top[u]);
        double tp;
        const double c = softmin2_cell(up, upn, cur, d, tp);
        up = upn;
        cur = c;
        bottom[u] = c;
        if (!REV) {
          if (STORE) __builtin_nontemporal_store(c, (u < 8 ? sp : sp8) + (u & 7) * dir);
          if (CKPT && band_ck && ckp) ckp[t] = c;
        } else if (!boundary) {
          const float ev = align_entry(xnm, rn[u], tp);
          dr[((t - lane) & (FR - 1)) * kFPitch + lane] = ev;
          if (ALIGN) {
            const int col = t - lane;
            if (alignp && col < M) alignp[M - 1 - col] = ev;
          }
        }
      }
    };
    if constexpr (SPLIT) {
      const bool want_align = REV && a.align != nullptr;
      if (t0 < 64) {
        if (want_align)
          run_steps(std::true_type{}, std::true_type{});
        else
          run_steps(std::true_type{}, std::false_type{});
      } else {
        if (want_align)
          run_steps(std::false_type{}, std::true_type{});
        else
          run_steps(std::false_type{}, std::false_type{});
      }
    } else {
      run_steps(std::true_type{}, std::true_type{});   // tests kept per step
    }
    if (lane == 0) lds_publish(&sh.dp_done, (unsigned)q + 1);

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
    if (top_ring && lane == 0) lds_publish(&sh.rd_in, umin_u((unsigned)t0 + kCH, Mu));
    if (direct_out) {
      stress_delay(5);
      if (lane == 63) {
        const int c0 = t0 - 63;                  // column of step t0
        if (c0 >= 0 && c0 + kCH <= M) {
#pragma unroll
          for (int u = 0; u < kCH; ++u)
            __hip_atomic_store(hout + c0 + u, bottom[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
#pragma unroll
          for (int u = 0; u < kCH; ++u)
            if (c0 + u >= 0 && c0 + u < M)
              __hip_atomic_store(hout + c0 + u, bottom[u], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else if (out_used) {
      const int cmax = t0 + kCH - 1 - 63;
      if (cmax >= kRingC) {
        const unsigned need = (unsigned)(cmax - kRingC + 1);
        if (seen_rd < need) seen_rd = lds_wait_ge(&sh.rd_out, need);
      }
      if (lane == 63) {
        // Same slot arithmetic as the unfused band waves (padded ring row).
        const int s0 = (t0 + kRingC - 63) & (kRingC - 1);
        double* rw = &sh.ring_out[s0];
#pragma unroll
        for (int u = 0; u < kCH; ++u) rw[u] = bottom[u];
        if (s0 + kCH > kRingC) sh.ring_out[0] = bottom[kRingC - s0];
        const int done = t0 + kCH - 63;
        lds_publish(&sh.wr_out, done <= 0 ? 0u : umin_u((unsigned)done, Mu));
      }
    }
  };
  for (int q = 0; q < qcount; q += 2) {
    chunk(q, rnA, rnB);
    if (q + 1 < qcount) chunk(q + 1, rnB, rnA);
  }
}

// ---------------------------------------------------------------------------
// Distance helper h of nh: blocks p = h, h+nh, ... (sweep columns [16p, 16p+16)).
// ---------------------------------------------------------------------------
template <bool REV, int NHC, int FR>
__device__ __forceinline__ void fused_dist_helper(const DPArgs& a, FusedShared& sh,
                                                  const float* xs, float* dr, int b, int h,
                                                  int nh, int lane) {
  const int64_t M = a.M, D = a.D;
  const int P = fused_pitch(D);
  const int qcount = (int)(sweep_steps(M) / kCH);
  const int r16 = lane & 15, kk = lane >> 4;
  const int steps4 = (int)((D + 3) / 4);
  const float* yb = a.y + (int64_t)b * M * D;
  // Row norms of the four 16-row tiles, accumulated exactly as the distance
  // kernel does (per lane over d = 4s + k, then across the four k lanes).
  double nxt[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    double p = 0.0;
    for (int s = 0; s < steps4; ++s) {
      const double v = (double)xs[(16 * ti + r16) * P + 4 * s + kk];
      p = fma(v, v, p);
    }
    p += __shfl_xor(p, 16, 64);
    p += __shfl_xor(p, 32, 64);
    nxt[ti] = p;
  }
  unsigned seen_dp = 0, seen_e = 0;
  for (int p = h; p < qcount; p += nh) {
    // Block p takes the slots of block p - R (R = FR / 16 blocks in the
    // ring): the band wave must be past it (its last reader is chunk
    // p - R + 4, i.e. dp_done >= p - R + 5) and, in the reverse sweep, the
    // chain-rule helpers must have released it (e_free >= p - R + 1).
    constexpr int R = FR / kCH;
    if (p >= R) {
      const unsigned need = (unsigned)(p - R + 5);
      if (seen_dp < need) seen_dp = lds_wait_ge(&sh.dp_done, need);
      if (REV && seen_e < (unsigned)(p - R + 1)) {
        unsigned m = ~0u;
        for (int c = 0; c < NHC; ++c)
          m = umin_u(m, lds_wait_ge(&sh.e_free[c], (unsigned)(p - R + 1)));
        seen_e = m;
      }
    }
    const int64_t sc = (int64_t)p * kCH + r16;      // sweep column of this lane
    const bool cok = sc < M;
    const int64_t oc = cok ? (REV ? M - 1 - sc : sc) : 0;
    const float* yr = yb + oc * D;
    v4d acc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) acc[ti] = (v4d){0.0, 0.0, 0.0, 0.0};
    double ny = 0.0;
    // y values in batches of kYB feature steps, all requested before the
    // batch's matrix instructions, so a batch costs one memory round trip
    // instead of one per step.  Full batches run unguarded; the last, partial
    // one skips the steps past D.
    auto batch = [&](int s0, auto guard) {
      float yv[kYB];
#pragma unroll
      for (int j = 0; j < kYB; ++j) {
        const int d = 4 * (s0 + j) + kk;
        yv[j] = yr[d < D ? d : D - 1];
      }
#pragma unroll
      for (int j = 0; j < kYB; ++j) {
        const int s = s0 + j;
        if (!decltype(guard)::value || s < steps4) {
          const int d = 4 * s + kk;
          const double bv = (d < D && cok) ? (double)yv[j] : 0.0;
          ny = fma(bv, bv, ny);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            const double av = (double)xs[(16 * ti + r16) * P + 4 * s + kk];
            acc[ti] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[ti], 0, 0, 0);
          }
        }
      }
    };
    int s0 = 0;
    for (; s0 + kYB <= steps4; s0 += kYB) batch(s0, std::false_type{});
    if (s0 < steps4) batch(s0, std::true_type{});
    ny += __shfl_xor(ny, 16, 64);
    ny += __shfl_xor(ny, 32, 64);
    float* col = dr + (int)(sc & (FR - 1)) * kFPitch;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = 4 * e + kk;  // fp64 16x16x4 accumulator row
        const double nxr = __shfl(nxt[ti], rl, 64);
        double v = nxr + ny - 2.0 * acc[ti][e];
        v = v > 0.0 ? v : 0.0;
        col[16 * ti + rl] = (float)v;
      }
    // Publish in block order.
    (void)lds_wait_ge(&sh.d_ready, (unsigned)p);
    if (lane == 0) lds_publish(&sh.d_ready, (unsigned)p + 1);
  }
}

// ---------------------------------------------------------------------------
// Chain-rule helper c of nhc (reverse sweep).  D is cut into slices of DC
// columns; when there are helpers to spare, the helpers of a slice (its
// "phases") take its blocks in turn (each keeps its part of dx; the others
// hand their parts over through LDS at the end, and the first adds them in
// phase order and writes dx).  The y rows of a helper's next block are requested while
// a block is processed and staged in the helper's LDS area `ys` (two
// blocks), so a block never waits on memory.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int chain_phases(int64_t D, int DC, int nhc) {
  const int nsl = (int)((D + DC - 1) / DC);
  const int nph = nhc / nsl;
  return nph < 1 ? 1 : nph;
}
// LDS floats for the dx hand-over between the helpers of a slice.
__host__ __device__ constexpr int chain_xch_floats(int64_t D, int DC, int nhc) {
  return (int)((D + DC - 1) / DC) * (chain_phases(D, DC, nhc) - 1) * 64 * (32 * (DC / 32) + 2);
}

template <int DC, int FR>
__device__ __forceinline__ void fused_chain_helper(const DPArgs& a, FusedShared& sh,
                                                   const float* xs, const float* dr,
                                                   float* ys, float* xch, int b, int band,
                                                   int c, int nhc, int lane) {
  constexpr int NT = DC / 32;
  constexpr int YP = DC + 2;            // staged row pitch
  constexpr int YL = 16 * DC / 64;      // staged values per lane per block
  const int64_t N = a.N, M = a.M, D = a.D;
  const int P = fused_pitch(D);
  const int qcount = (int)(sweep_steps(M) / kCH);
  const int64_t r0 = a.row0 + (int64_t)band * 64;
  const int nsl = (int)((D + DC - 1) / DC);
  const int nph = chain_phases(D, DC, nhc);
  const int slice = c % nsl, phase = c / nsl;
  const int64_t dbeg = (int64_t)slice * DC;
  const bool want_gx = a.gx != nullptr, want_gy = a.gy != nullptr;
  if ((!want_gx && !want_gy) || phase >= nph || dbeg >= D) {
    if (lane == 0) lds_publish(&sh.e_free[c], (unsigned)qcount);
    return;
  }
  // Blocks of the other phase are never this helper's to release.
  if (phase > 0 && lane == 0) lds_publish(&sh.e_free[c], (unsigned)phase);
  const int64_t dend = dbeg + DC < D ? dbeg + DC : D;
  const float g2 = 2.f * a.gl[b];
  const float* yb = a.y + (int64_t)b * M * D;
  const int r32 = lane & 31, h = lane >> 5;
  const int r16 = lane & 15, kk = lane >> 4;
  v16f gxa[2][NT];
  float rsum[2] = {0.f, 0.f};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) gxa[rt][t][e] = 0.f;

  // Block p's y rows (sweep columns 16p .. 16p+15, columns dbeg .. dbeg+DC-1
  // of D; rows past M and columns past D are clamped copies, multiplied by
  // zero alignment entries or never written out).
  float yreg[YL];
  auto load_y = [&](int p) {
#pragma unroll
    for (int k = 0; k < YL; ++k) {
      const int idx = lane + 64 * k;
      const int64_t sc = (int64_t)p * kCH + idx / DC;
      const int64_t oc = sc < M ? M - 1 - sc : 0;
      const int64_t dc = dbeg + idx % DC;
      yreg[k] = yb[oc * D + (dc < D ? dc : D - 1)];
    }
  };
  auto stage_y = [&](int k) {             // k: the helper's own block count
    float* yd = ys + (chain_y_bufs(DC) == 2 ? (k & 1) : 0) * 16 * YP;
#pragma unroll
    for (int k = 0; k < YL; ++k) {
      const int idx = lane + 64 * k;
      yd[(idx / DC) * YP + idx % DC] = yreg[k];
    }
  };

  const int nreal = (int)((M + kCH - 1) / kCH);
  load_y(phase);
  stage_y(0);
  unsigned seen_dp = 0;
  for (int p = phase, k = 0; p < nreal; p += nph, ++k) {
    const bool more = p + nph < nreal;
    if (more) load_y(p + nph);
    // Block p is complete once the band wave has finished chunk p+4 (the
    // last chunk completes every remaining block).
    const unsigned need = umin_u((unsigned)p + 5, (unsigned)qcount);
    if (seen_dp < need) seen_dp = lds_wait_ge(&sh.dp_done, need);
    const int64_t c0 = (int64_t)p * kCH;
    const float* yc = ys + (chain_y_bufs(DC) == 2 ? (k & 1) : 0) * 16 * YP;
    if (want_gx) {
      // dx += E[64 x 16] . Y[16 x DC] on v_mfma_f32_32x32x2_f32.  Up to
      // DC = 64 the block's E entries are read as one batch (unconditional
      // reads, masked after), so the LDS latency is paid once per block, not
      // once per product; the widest slice keeps per-product reads (its
      // accumulators leave no registers for the batch).
      constexpr bool kBatch = NT <= 2;
      float ev[8][2];
      if (kBatch) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float* ecol = dr + (int)((c0 + 2 * s + h) & (FR - 1)) * kFPitch;
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) ev[s][rt] = ecol[32 * rt + r32];
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int cl = 2 * s + h;                 // column of the block
        const bool cok = c0 + cl < M;
        const float* ecol = dr + (int)((c0 + cl) & (FR - 1)) * kFPitch;
        float av[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int row = 32 * rt + r32;
          const bool ok = cok && r0 + row < N;
          av[rt] = kBatch ? (ok ? ev[s][rt] : 0.f) : (ok ? ecol[row] : 0.f);
          rsum[rt] += av[rt];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float bv = yc[cl * YP + 32 * t + r32];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            gxa[rt][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[rt], bv, gxa[rt][t], 0, 0, 0);
        }
      }
    }
    v4f acc[2 * NT];
    float cs = 0.f;
    if (want_gy) {
      // dy[16 columns] += 2g (colsum(E) y - E^T . X[64 x DC]) on
      // v_mfma_f32_16x16x4_f32, added atomically (other bands add too).
#pragma unroll
      for (int t = 0; t < 2 * NT; ++t) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
      const bool cok = c0 + r16 < M;
      const float* ecol = dr + (int)((c0 + r16) & (FR - 1)) * kFPitch;
      // Up to DC = 64, E and the x operands are read as one batch; columns
      // of D past dend then read a clamped in-range entry whose products are
      // never written out.
      constexpr bool kBatchY = NT <= 2;
      float ev[16];
      int xo[2 * NT];
#pragma unroll
      for (int t = 0; t < 2 * NT; ++t) {
        const int64_t dc = dbeg + 16 * t + r16;
        xo[t] = (int)(dc < D ? dc : D - 1);
      }
      if (kBatchY) {
#pragma unroll
        for (int s = 0; s < 16; ++s) ev[s] = ecol[4 * s + kk];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int row = 4 * s + kk;
        const bool ok = cok && r0 + row < N;
        const float av = kBatchY ? (ok ? ev[s] : 0.f) : (ok ? ecol[row] : 0.f);
        cs += av;
#pragma unroll
        for (int t = 0; t < 2 * NT; ++t) {
          const int64_t dc = dbeg + 16 * t + r16;
          const float bv = kBatchY ? xs[row * P + xo[t]] : (dc < dend ? xs[row * P + dc] : 0.f);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[t], 0, 0, 0);
        }
      }
      cs += __shfl_xor(cs, 16, 64);
      cs += __shfl_xor(cs, 32, 64);
    }
    // With two staging slots the next block's y rows go into the other one
    // (last read in the block before this one) before this block's atomics
    // are issued.
    if (chain_y_bufs(DC) == 2 && more) stage_y(k + 1);
    if (want_gy) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ci = 4 * kk + e;  // fp32 16x16x4 accumulator row
        const float csum = __shfl(cs, ci, 64);
        const int64_t scol = c0 + ci;
        if (scol < M) {
          const int64_t oc = M - 1 - scol;
          float* gyr = a.gy + ((int64_t)b * M + oc) * D;
#pragma unroll
          for (int t = 0; t < 2 * NT; ++t) {
            const int64_t dc = dbeg + 16 * t + r16;
            if (dc < dend)
              atomicAdd(gyr + dc, g2 * (csum * yc[ci * YP + 16 * t + r16] - acc[t][e]));
          }
        }
      }
    }
    // With one slot they replace this block's rows after its last reads
    // (the LDS performs one wave's operations in order).
    if (chain_y_bufs(DC) == 1 && more) stage_y(k + 1);
    if (lane == 0) lds_publish(&sh.e_free[c], umin_u((unsigned)(p + nph), (unsigned)qcount));
  }
  if (lane == 0) lds_publish(&sh.e_free[c], (unsigned)qcount);
  if (want_gx && nph > 1) {
    // The other helpers of the slice hand their parts of dx (products and
    // row sums) to the first, which adds them to its own in phase order.
    constexpr int XW = 32 * NT + 2;
    float* const xs0 = xch + slice * (nph - 1) * 64 * XW;
    if (phase > 0) {
      float* xd = xs0 + (phase - 1) * 64 * XW;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) xd[((rt * NT + t) * 16 + e) * 64 + lane] = gxa[rt][t][e];
        xd[(32 * NT + rt) * 64 + lane] = rsum[rt];
      }
      if (lane == 0) lds_publish(&sh.x_done[c], 1u);
      return;
    }
    for (int f = 1; f < nph; ++f) {
      const float* xd = xs0 + (f - 1) * 64 * XW;
      (void)lds_wait_ge(&sh.x_done[slice + f * nsl], 1u);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) gxa[rt][t][e] += xd[((rt * NT + t) * 16 + e) * 64 + lane];
        rsum[rt] += xd[(32 * NT + rt) * 64 + lane];
      }
    }
  }

  if (want_gx) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float rsf = rsum[rt] + __shfl_xor(rsum[rt], 32, 64);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rowi = 8 * (e >> 2) + 4 * h + (e & 3);
        const float rs = __shfl(rsf, rowi, 64);
        const int64_t si = r0 + 32 * rt + rowi;
        if (si < N) {
          const int64_t orr = N - 1 - si;
          float* gxr = a.gx + ((int64_t)b * N + orr) * D;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int64_t dc = dbeg + 32 * t + r32;
            if (dc < dend)   // device-coherent (see release_ctrl)
              __hip_atomic_store(gxr + dc, g2 * (rs * xs[(32 * rt + rowi) * P + dc] - gxa[rt][t][e]),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One band per workgroup.  Waves: 0 = band wave, then HD distance helpers,
// then HC chain-rule helpers (reverse only), then the hand-off wave.
// Tickets give bands in order, so a band waits only on a smaller ticket.
// INFER: the forward sweep for the loss alone: no state is stored, and the
// rows handed between bands are either whole (hcols = 0) or global rings of
// hcols columns; with rings tickets run pair by pair (see above).
// ---------------------------------------------------------------------------
template <bool REV, bool INFER, bool CKPT, int HD, int HC, int DC, int FR>
__global__ __launch_bounds__((HD + HC + 2) * 64) void k_dp_fused(DPArgs a, unsigned hcols) {
  extern __shared__ float smem[];
  __shared__ FusedShared sh;
  constexpr int kIO = HD + HC + 1;
  constexpr int kNW = HD + HC + 2;
  const int lane = threadIdx.x & 63;
  // Role of each wave: 0 the band wave, 1..HD the distance helpers, then the
  // chain-rule helpers, kIO the hand-off wave.  A workgroup's waves go to
  // the CU's four SIMDs in turn, so wave 4 shares the band wave's SIMD: in a
  // workgroup of more than five waves it takes the light hand-off role and
  // the helpers go to the other SIMDs (fused reverse, B=32, N=M=512, D=64:
  // 190-201 -> 177 us; 32 x 256^2, D=64: 96-115 -> 87 us).
  const int wi = threadIdx.x >> 6;
  const int w = (kNW > 5 && wi == 4) ? kIO : ((kNW > 5 && wi == kIO) ? 4 : wi);
  if (threadIdx.x == 0) sh.ticket = atomicAdd(&a.ctrl[0], 1u);
  if (threadIdx.x == 0) {
    launch_shared_init(a);
    sh.wr_in = sh.rd_in = sh.wr_out = sh.rd_out = 0u;
    sh.d_ready = sh.dp_done = 0u;
    for (int c = 0; c < kRevHelpCMax; ++c) sh.e_free[c] = sh.x_done[c] = 0u;
  }
  __syncthreads();
  const unsigned ticket = sh.ticket;
  // Pair-major tickets with ring hand-off (a band may wait on the one below),
  // band-major otherwise (a band waits only on the one above).
  const bool pair_major = INFER && hcols != 0;
  const int band = pair_major ? (int)(ticket % (unsigned)a.nseg) : (int)(ticket / (unsigned)a.B);
  const int b = pair_major ? (int)(ticket / (unsigned)a.nseg) : (int)(ticket % (unsigned)a.B);
  const int64_t N = a.N, D = a.D;
  const int P = fused_pitch(D);
  float* xs = smem;
  float* dr = smem + 64 * P;

  // x rows of this band in sweep order, zero-padded to P columns.
  const float* xb = a.x + (int64_t)b * N * D;
  const int64_t r0 = a.row0 + (int64_t)band * 64;
  for (int idx = threadIdx.x; idx < 64 * P; idx += blockDim.x) {
    const int rr = idx / P, d = idx - rr * P;
    const int64_t si = r0 + rr;
    const bool ok = si < N && d < D;
    const int64_t orr = si < N ? (REV ? N - 1 - si : si) : 0;
    xs[idx] = ok ? xb[orr * D + d] : 0.f;
  }
  __syncthreads();

  if (w == 0) {
    fused_band<REV, !INFER, CKPT, (HD + HC + 2 <= 8), FR>(a, sh, dr, b, band, lane);
  } else if (w <= HD) {
    fused_dist_helper<REV, HC, FR>(a, sh, xs, dr, b, w - 1, HD, lane);
  } else if (w < kIO) {
    if (REV) {
      const int c = w - 1 - HD;
      float* ys = dr + FR * kFPitch + c * chain_y_floats(DC);
      float* xch = dr + FR * kFPitch + HC * chain_y_floats(DC);
      fused_chain_helper<DC, FR>(a, sh, xs, dr, ys, xch, b, band, c, HC, lane);
    }
  } else {
    const int64_t pb = (int64_t)b * a.nseg;
    const int64_t sin = pb + (band > 0 ? band - 1 : 0), sout = pb + band;
    const int64_t row = hcols ? hcols : a.M;   // doubles per hand-off row
    GlobalRow gr{0u, nullptr, nullptr};
    if (INFER && hcols) {
      // Fetched counts follow the progress counts in the control words.
      unsigned* fetched = a.ctrl + 2 + (int64_t)a.B * a.nseg;
      gr = GlobalRow{hcols, fetched + pb + band + 1, fetched + pb + band};
    }
    // A range launch takes its first band's top row complete from top_row
    // and hands its last band's bottom row out through bot_row.
    const bool ext_in = band == 0 && a.top_row != nullptr;
    const bool ext_out = band + 1 == a.nseg && a.bot_row != nullptr;
    if (!(INFER && hcols)) {
      gr.valid_in = a.hvalid != 0 && !ext_in;
      gr.valid_out = a.hvalid != 0 && !ext_out;
    }
    const bool direct_out = a.hvalid != 0 && !ext_out;   // the band wave writes the row
    // (for band + 1 < nseg, ext_out is false: the band wave's own choice)
    segment_io_wave(band > 0 || ext_in, (band + 1 < a.nseg && !direct_out) || ext_out,
                    ext_in ? a.full_word : a.ctrl + 2 + sin,
                    ext_out ? a.sink_word : a.ctrl + 2 + sout,
                    ext_in ? a.top_row + (int64_t)b * a.top_ld : a.H + sin * row,
                    ext_out ? a.bot_row + (int64_t)b * a.M : a.H + sout * row, sh.ring_in,
                    &sh.wr_in, &sh.rd_in, sh.ring_out, &sh.wr_out, &sh.rd_out,
                    (unsigned)a.M, lane, gr);
  }
  // The alignment-matrix output is written with ordinary stores.
  release_ctrl(a.ctrl, (INFER && hcols ? 2 : 1) * (int64_t)a.B * a.nseg,
               !(REV && a.align != nullptr));
}

template <bool REV, bool INFER, bool CKPT, int HD, int HC, int DC, int FR>
static hipError_t launch_fused_ring(const DPArgs& a, hipStream_t s, unsigned hcols,
                                    size_t lds) {
  auto kern = k_dp_fused<REV, INFER, CKPT, HD, HC, DC, FR>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)a.B * (unsigned)a.nseg;
  TimedLaunch timed_(INFER ? "dp_infer" : (REV ? "dp_fused_rev" : "dp_fused_fwd"), s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3((HD + HC + 2) * 64), lds, s, a, hcols);
  return hipGetLastError();
}

// Largest dynamic LDS a workgroup may take next to the static FusedShared
// (gfx950: 160 KiB per workgroup).
static size_t fused_lds_limit() {
  int dev = 0, lim = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    lim = 160 * 1024;
  return (size_t)lim > sizeof(FusedShared) ? (size_t)lim - sizeof(FusedShared) : 0;
}

// The ring of 16 blocks lets the distance helpers run up to 12 blocks
// ahead of the band wave, and in the reverse sweep lets a block's slot wait
// for the chain-rule helpers that long: with 8 blocks, a helper's block
// (y loads and fp64 MFMAs, ~4.4 us at D = 64) plus the chain-rule helpers'
// release of the slot did not fit in the four chunks of slack, and the band
// wave waited ~1 us per chunk for distances.  Measured (rocprof, fused
// reverse / forward, us, 8 -> 16 blocks): B=32, N=M=512, D=64 224.6 / 129.2
// -> 189.4 / 125.9; 32 x 256^2, D=128 155.7 / 102.2 -> 130.9 / 91.2;
// 32 x 4096 x 1000, D=128 2623 / 1583 -> 2556 / 1537; inference at B=32,
// N=M=512 124.2 -> 120.0.
template <bool REV, bool INFER, bool CKPT, int HD, int HC, int DC>
static hipError_t launch_fused_one(const DPArgs& a, hipStream_t s, unsigned hcols = 0) {
  static_assert(HC <= kRevHelpCMax, "chain-rule helpers");
  const size_t lds = fused_lds_bytes(a.D, REV ? DC : 0, HC, kFR) +
                     (REV ? (size_t)chain_xch_floats(a.D, DC, HC) * 4 : 0);
  if (lds > fused_lds_limit()) return hipErrorNotSupported;   // see fused_lds_fits
  return launch_fused_ring<REV, INFER, CKPT, HD, HC, DC, kFR>(a, s, hcols, lds);
}

// Every D the fused kernels take fits the 160 KiB of LDS of a gfx950
// workgroup with the full ring: the forward's x rows and ring, and the
// reverse's chain-rule helpers (DC = 32 up to D = 128, then 64) on top.
constexpr bool fused_lds_fits() {
  for (int64_t D = 1; D <= kFusedMaxD; ++D) {
    const int DC = D <= 4 * 32 ? 32 : 64;
    const size_t rev = fused_lds_bytes(D, DC, kRevHelpCMax, kFR) +
                       (size_t)chain_xch_floats(D, DC, kRevHelpCMax) * 4;
    const size_t fwd = fused_lds_bytes(D, 0, 0, kFR);
    if (fwd + sizeof(FusedShared) > 160 * 1024 || rev + sizeof(FusedShared) > 160 * 1024)
      return false;
  }
  return true;
}
static_assert(fused_lds_fits(), "fused workgroup LDS");

hipError_t launch_dp_fused(const DPArgs& a, bool reverse, hipStream_t s) {
  if (fused_bands_per_wg(a.D) == 0) return hipErrorNotSupported;
  // Forward: the distance helpers alone keep the ring ahead of the band
  // wave.  Up to D = 64 three do (six change nothing); beyond, six, two
  // on each SIMD but the band wave's (rocprof, us, three -> six helpers:
  // 32 x 256^2, D=128 91 -> 83, D=256 146 -> 131; 32 x 1024^2, D=128
  // 452 -> 402; 32 x 4096 x 1000, D=128 1541 -> 1356; four or five
  // helpers gain less or lose).
  if (!reverse) {
    if (a.D > 64) return launch_fused_one<false, false, false, kFwdHelpDWide, 0, 32>(a, s);
    return launch_fused_one<false, false, false, kFwdHelpD, 0, 32>(a, s);
  }
  // The reverse workgroup: the band wave, HD distance helpers, HC chain-rule
  // helpers on slices of DC columns of D (32 up to D = 128, then 64: wider
  // slices would not keep their accumulators in registers) and the hand-off
  // wave.  Where there are fewer slices than helpers, the helpers of a slice
  // take its blocks in turn.  Per range of D (rocprof, fused reverse, us):
  //   D <= 32 (one slice):       HD 3, HC 2; two chain-rule helpers keep up
  //                              (32 x 512^2, D=16: 163 with HD 2, HC 4 ->
  //                              153; 32 x 1024^2, D=16: 391 -> 363)
  //   D <= 64 (two slices):      HD 2, HC 4; two chain-rule helpers fall
  //                              behind (B=32, N=M=512: 177 -> 212 with
  //                              HD 3, HC 2)
  //   D <= 96 (three slices):    HD 3, HC 3, eight waves, each distance
  //                              helper beside a chain-rule helper (32 x
  //                              256^2, D=80: 129 with HD 3, HC 4 -> 106;
  //                              32 x 1024^2, D=72: 655 -> 603)
  //   D <= 128 (four slices):    HD 3, HC 4 (32 x 1024^2: 826 against 891
  //                              with HD 2)
  //   D <= 192 (three slices):   HD 3, HC 3 (32 x 256^2, D=160: 219 with
  //                              HD 2, HC 4 -> 172)
  //   D <= 256 (four slices):    HD 2, HC 4; nine waves would leave the
  //                              64-column helpers too few registers
  if (a.D <= 32)
    return launch_fused_one<true, false, false, kRevHelpD + 1, 2, 32>(a, s);
  if (a.D <= 2 * 32)
    return launch_fused_one<true, false, false, kRevHelpD, kRevHelpCMax, 32>(a, s);
  if (a.D <= 3 * 32)
    return launch_fused_one<true, false, false, kRevHelpD + 1, 3, 32>(a, s);
  if (a.D <= 4 * 32)
    return launch_fused_one<true, false, false, kRevHelpD + 1, kRevHelpCMax, 32>(a, s);
  if (a.D <= 3 * 64)
    return launch_fused_one<true, false, false, kRevHelpD + 1, 3, 64>(a, s);
  return launch_fused_one<true, false, false, kRevHelpD, kRevHelpCMax, 64>(a, s);
}

hipError_t launch_fused_range(const DPArgs& a, bool reverse, hipStream_t s) {
  // Forward ranges start their state rows at their first sweep row, so a
  // lane's storage row keeps the lane's position in its band.
  if (!reverse && a.row0 != a.xrow0) return hipErrorInvalidValue;
  if (reverse && (a.row0 & 63) != 0) return hipErrorInvalidValue;
  return launch_dp_fused(a, reverse, s);
}

hipError_t launch_infer(const DPArgs& a, unsigned hcols, hipStream_t s) {
  if (fused_bands_per_wg(a.D) == 0) return hipErrorNotSupported;
  // The distance helpers as in the training forward (launch_dp_fused).
  if (a.D > 64) {
    if (a.ckpt) return launch_fused_one<false, true, true, kFwdHelpDWide, 0, 32>(a, s, hcols);
    return launch_fused_one<false, true, false, kFwdHelpDWide, 0, 32>(a, s, hcols);
  }
  if (a.ckpt) return launch_fused_one<false, true, true, kFwdHelpD, 0, 32>(a, s, hcols);
  return launch_fused_one<false, true, false, kFwdHelpD, 0, 32>(a, s, hcols);
}

}  // namespace sdtw

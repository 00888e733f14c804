// Fused-distance wavefront kernels (gfx950): no B x N x M distance tensor.
//
// The README "SoftDTW-CUDA (PyTorch + Numba)" ("Fused Mode": no distance
// tensor; "Limitations": squared Euclidean only) and the review page
// "SoftDTW-CUDA-Torch" ("Proposed method": distances recomputed on the fly)
// describe a mode that never materialises Dist.  Here each band (64 rows)
// keeps its x rows in LDS and, at every chunk of 16 steps, recomputes the
// 64 x 16 block of distances the wavefront is about to enter with fp64 MFMA
// (the same operations, in the same order, as the distance kernel, so fused
// and unfused distances are bit-identical) into an 80-column LDS ring that
// the steps read.
//
// The reverse sweep replaces every ring entry by its alignment value E once
// the cell is done; when a 16-column block of the band is complete (four
// chunks later) it contributes, on fp32 MFMA,
//   dx[rows of the band] += 2g (rowsum(E) x - E . Y)    (kept in registers),
//   dy[16 columns]       += 2g (colsum(E) y - E^T . X)  (atomic adds, the
//                                                       bands share columns),
// so neither Dist nor E ever reaches global memory.  The gradient columns of
// D are covered in slices of 32*NT per launch.
#include "sdtw_dp_common.h"

namespace sdtw {

constexpr int kDRing = 80;   // distance/E ring columns per band (79 are live)
constexpr int kDPitch = 66;  // floats per ring column: 64 rows + 2 (LDS banks)

__host__ __device__ inline int fused_pitch(int64_t D) { return (int)(((D + 3) / 4) * 4 + 4); }

size_t fused_lds_bytes(int W, int64_t D) {
  return (size_t)W * (64 * (size_t)fused_pitch(D) + (size_t)kDRing * kDPitch) * 4;
}

// Bands per workgroup for the fused kernels: as many as the LDS holds (the
// x rows of each band plus its ring), 0 when D is beyond what they support.
int fused_bands_per_wg(int64_t D) {
  if (D < 1 || D > kFusedMaxD) return 0;
  const size_t static_lds = 3 * kRing * 8 + 64;
  for (int W : {4, 2, 1})
    if (fused_lds_bytes(W, D) + static_lds <= 163840) return W;
  return 0;
}

template <int NT>
struct GradAcc {
  v16f x[2][NT];
  float rsum[2];
};

template <bool REV, int W, int KD, int NT>
__global__ __launch_bounds__(W * 64) void k_dp_fused(DPArgs a, int64_t d0) {
  extern __shared__ float smem[];
  __shared__ double ring[W > 1 ? W - 1 : 1][kRing];
  __shared__ unsigned s_ticket;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.ctrl[0], 1u);
  __syncthreads();
  const unsigned ticket = s_ticket;
  const int seg = (int)(ticket / (unsigned)a.B);
  const int b = (int)(ticket % (unsigned)a.B);

  const int64_t N = a.N, M = a.M, D = a.D, S = a.S;
  const int P = fused_pitch(D);
  const int band = seg * W + w;
  const int nb_seg = min(W, a.nbands - seg * W);
  const bool active = w < nb_seg;
  const int64_t r0 = (int64_t)(active ? band : 0) * 64;
  const int64_t i = r0 + lane;
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
  double* rsk = a.R;
  const double k2 = a.k2;
  const double xnm = REV ? a.loss64[b] : 0.0;
  float* xs = smem + w * 64 * P;
  float* dr = smem + W * 64 * P + w * kDRing * kDPitch;
  const float* xb = a.x + (int64_t)b * N * D;
  const float* yb = a.y + (int64_t)b * M * D;

  // x rows of this band in sweep order, zero-padded to P columns.
  if (active) {
    for (int rr = 0; rr < 64; ++rr) {
      const int64_t si = r0 + rr;
      const bool ok = si < N;
      const int64_t orr = ok ? (REV ? N - 1 - si : si) : 0;
      for (int d = lane; d < P; d += 64) xs[rr * P + d] = (ok && d < D) ? xb[orr * D + d] : 0.f;
    }
  }
  // Row norms of the four 16-row tiles, accumulated exactly as the distance
  // kernel does (per lane over d = 4s + k, then across the four k lanes).
  const int r16 = lane & 15, kk = lane >> 4;
  const int steps4 = (int)((D + 3) / 4);
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

  // y operand of the next distance block, fetched one chunk ahead.
  float yq[KD];
  auto fetch_y = [&](int q) {
    const int64_t sc = (int64_t)q * kCH + r16;
    const bool cok = sc < M;
    const int64_t oc = cok ? (REV ? M - 1 - sc : sc) : 0;
    const float* yr = yb + oc * D;
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      const int d = 4 * s + kk;
      yq[s] = yr[d < D ? d : D - 1];
    }
  };
  // Distances of sweep columns [16q, 16q+16) for the band's 64 rows.
  auto dist_block = [&](int q) {
    const int64_t c0 = (int64_t)q * kCH;
    const bool cok = c0 + r16 < M;
    v4d acc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) acc[ti] = (v4d){0.0, 0.0, 0.0, 0.0};
    double ny = 0.0;
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      if (s < steps4) {
        const bool vd = 4 * s + kk < D;
        const double bv = (vd && cok) ? (double)yq[s] : 0.0;
        ny = fma(bv, bv, ny);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const double av = (double)xs[(16 * ti + r16) * P + 4 * s + kk];
          acc[ti] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[ti], 0, 0, 0);
        }
      }
    }
    ny += __shfl_xor(ny, 16, 64);
    ny += __shfl_xor(ny, 32, 64);
    const int slot = (int)((c0 + r16) % kDRing);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = 4 * e + kk;  // fp64 16x16x4 accumulator row
        const double nxr = __shfl(nxt[ti], rl, 64);
        double v = nxr + ny - 2.0 * acc[ti][e];
        v = v > 0.0 ? v : 0.0;
        dr[slot * kDPitch + 16 * ti + rl] = (float)v;
      }
  };

  GradAcc<NT> g;
  if (REV) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      g.rsum[rt] = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) g.x[rt][t][e] = 0.f;
    }
  }
  const float g2 = REV ? 2.f * a.gl[b] : 0.f;
  const bool want_gx = REV && a.gx != nullptr;
  const bool want_gy = REV && a.gy != nullptr;
  const int64_t dlim = d0 + 32 * NT < D ? d0 + 32 * NT : D;

  // Contributions of the completed sweep columns [16p, 16p+16).
  auto grad_block = [&](int p) {
    const int64_t c0 = (int64_t)p * kCH;
    if (want_gx) {
      const int c = lane & 31, h = lane >> 5;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int64_t sc = c0 + 2 * s + h;
        const bool cok = sc < M;
        const int64_t oc = cok ? (REV ? M - 1 - sc : sc) : 0;
        const int slot = (int)(sc % kDRing);
        float av[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int row = 32 * rt + c;
          const bool ok = cok && (r0 + row < N);
          av[rt] = ok ? dr[slot * kDPitch + row] : 0.f;
          g.rsum[rt] += av[rt];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int64_t dc = d0 + 32 * t + c;
          const float bv = yb[oc * D + (dc < D ? dc : D - 1)];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            g.x[rt][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[rt], bv, g.x[rt][t], 0, 0, 0);
        }
      }
    }
    if (want_gy) {
      v4f acc[2 * NT];
#pragma unroll
      for (int t = 0; t < 2 * NT; ++t) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
      const int64_t sc = c0 + r16;
      const bool cok = sc < M;
      const int slot = (int)(sc % kDRing);
      float cs = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int row = 4 * s + kk;
        const bool ok = cok && (r0 + row < N);
        const float av = ok ? dr[slot * kDPitch + row] : 0.f;
        cs += av;
#pragma unroll
        for (int t = 0; t < 2 * NT; ++t) {
          const int64_t dc = d0 + 16 * t + r16;
          const float bv = dc < D ? xs[row * P + dc] : 0.f;
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[t], 0, 0, 0);
        }
      }
      cs += __shfl_xor(cs, 16, 64);
      cs += __shfl_xor(cs, 32, 64);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ci = 4 * kk + e;  // fp32 16x16x4 accumulator row
        const float csum = __shfl(cs, ci, 64);
        const int64_t scol = c0 + ci;
        if (scol < M) {
          const int64_t oc = REV ? M - 1 - scol : scol;
          float* gyr = a.gy + ((int64_t)b * M + oc) * D;
          const float* yr = yb + oc * D;
#pragma unroll
          for (int t = 0; t < 2 * NT; ++t) {
            const int64_t dc = d0 + 16 * t + r16;
            if (dc < dlim) atomicAdd(gyr + dc, g2 * (csum * yr[dc] - acc[t][e]));
          }
        }
      }
    }
  };

  double cur = kBig;
  double up = (lane == 0 && r0 == 0) ? 0.0 : kBig;
  unsigned avail = 0;
  const int64_t lastrow = N - 1;
  const bool has_last = !REV && active && (lastrow >> 6) == band;
  const int64_t tlast = M - 1 + (lastrow & 63);
  const int qlast = (int)(tlast / kCH), ulast = (int)(tlast % kCH);
  float* alignp = (REV && a.align && row_ok) ? a.align + ((int64_t)b * N + (N - 1 - i)) * M : nullptr;

  double rn[kCH], tn[kCH];
  auto load_x = [&](int qq, double (&R_)[kCH]) {
#pragma unroll
    for (int u = 0; u < kCH; ++u) R_[u] = rsk[cu.base + ((int64_t)qq * kCH + u) * cu.dir];
  };
  auto await_cols = [&](int64_t need_) {
    const unsigned need = (unsigned)need_;
    if (avail < need) avail = await_progress(prog_in, need);
  };
  auto load_top = [&](int qq, double (&T_)[kCH]) {
#pragma unroll
    for (int u = 0; u < kCH; ++u) {
      const int64_t col = (int64_t)qq * kCH + u;
      T_[u] = Hin[col < M ? col : M - 1];
    }
  };

  if (active) {
    if (REV) load_x(0, rn);
    fetch_y(0);
  }
  if (consume_global) {
    await_cols(imin64(M, kCH + kSlack));
    load_top(0, tn);
  }
  __builtin_amdgcn_s_waitcnt(0);

  for (int Q = 0; Q < qtot; ++Q) {
    const int q = Q - kLag * w;
    if (active && q >= 0 && q < qcount) {
      const int64_t t0 = (int64_t)q * kCH;
      dist_block(q);
      const bool more = q + 1 < qcount;
      double rn2[kCH], tn2[kCH];
      if (more) {
        fetch_y(q + 1);
        if (REV) load_x(q + 1, rn2);
        if (consume_global) {
          await_cols(imin64(M, t0 + 2 * kCH));
          load_top(q + 1, tn2);
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
      int slot = (int)((t0 - lane + 64 * kDRing) % kDRing);
#pragma unroll
      for (int u = 0; u < kCH; ++u) {
        const int64_t t = t0 + u;
        float* cellp = dr + slot * kDPitch + lane;
        const double d = row_ok ? (double)(*cellp) * k2 : 0.0;
        const double upn = wave_shr1(cur, top[u]);
        const double diag = up;
        up = upn;
        const double tpart = softmin2_part(diag, upn, cur);
        double c = tpart + d;
        c = (t - lane < 0) ? kBig : c;
        cur = c;
        bottom[u] = c;
        if (!REV) {
          __builtin_nontemporal_store(c, rsk + cu.base + t * cu.dir);
        } else {
          const float ev = align_entry(xnm, rn[u], tpart);
          *cellp = ev;
          const int64_t col = t - lane;
          if (alignp && col >= 0 && col < M) alignp[M - 1 - col] = ev;
        }
        slot = slot + 1 == kDRing ? 0 : slot + 1;
      }

      // Block p is complete once lane 63 has passed column 16p+15, i.e. by
      // the end of chunk p+4; the last chunk completes every remaining block.
      if (REV) {
        const int plast = (int)((M - 1) / kCH);
        const int phi = (q == qcount - 1) ? plast : q - 4;
        for (int p = q - 4 < 0 ? 0 : q - 4; p <= phi; ++p) grad_block(p);
      }

      if (has_last && q == qlast) {
        double v = 0.0;
#pragma unroll
        for (int u = 0; u < kCH; ++u) v = (u == ulast) ? bottom[u] : v;
        if (lane == (int)(lastrow & 63)) {
          a.loss64[b] = v;
          a.loss[b] = (float)(v * a.g_ln2);
        }
      }
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
      if (more) {
#pragma unroll
        for (int u = 0; u < kCH; ++u) {
          if (REV) rn[u] = rn2[u];
          if (consume_global) tn[u] = tn2[u];
        }
      }
    }
    __syncthreads();
  }

  // dx of the band's rows for this slice of D.
  if (want_gx && active) {
    const int c = lane & 31, h = lane >> 5;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float rsf = g.rsum[rt] + __shfl_xor(g.rsum[rt], 32, 64);
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
            const int64_t dc = d0 + 32 * t + c;
            if (dc < dlim) gxr[dc] = g2 * (rs * xs[(32 * rt + rowi) * P + dc] - g.x[rt][t][e]);
          }
        }
      }
    }
  }
  release_ctrl(a.ctrl, (int64_t)a.B * a.nseg);
}

template <bool REV, int W, int KD, int NT>
static hipError_t launch_fused_one(const DPArgs& a, int64_t d0, hipStream_t s) {
  auto kern = k_dp_fused<REV, W, KD, NT>;
  const size_t lds = fused_lds_bytes(W, a.D);
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)a.B * (unsigned)a.nseg;
  TimedLaunch timed_(REV ? "dp_fused_rev" : "dp_fused_fwd", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(W * 64), lds, s, a, d0);
  return hipGetLastError();
}

hipError_t launch_dp_fused(const DPArgs& a, bool reverse, hipStream_t s) {
  const int W = fused_bands_per_wg(a.D);
  if (W == 0) return hipErrorNotSupported;
  const int kd = a.D <= 64 ? 16 : (a.D <= 128 ? 32 : 64);  // ceil(D/4) <= kd
  if (!reverse) {
    if (W == 4) return launch_fused_one<false, 4, 16, 1>(a, 0, s);
    if (W == 2 && kd == 32) return launch_fused_one<false, 2, 32, 1>(a, 0, s);
    if (W == 2) return launch_fused_one<false, 2, 64, 1>(a, 0, s);
    return launch_fused_one<false, 1, 64, 1>(a, 0, s);
  }
  // Reverse: one sweep per slice of D (32 * NT columns of the gradients).
  const int nt = a.D <= 32 ? 1 : (a.D <= 64 ? 2 : (a.D <= 96 ? 3 : 4));
  for (int64_t d0 = 0; d0 < a.D; d0 += 32 * nt) {
    hipError_t e;
    if (W == 4)
      e = nt == 1 ? launch_fused_one<true, 4, 16, 1>(a, d0, s)
                  : launch_fused_one<true, 4, 16, 2>(a, d0, s);
    else if (W == 2 && kd == 32)
      e = nt == 3 ? launch_fused_one<true, 2, 32, 3>(a, d0, s)
                  : launch_fused_one<true, 2, 32, 4>(a, d0, s);
    else if (W == 2)
      e = launch_fused_one<true, 2, 64, 4>(a, d0, s);
    else
      e = launch_fused_one<true, 1, 64, 4>(a, d0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sdtw

// C ABI of the gfx950 Soft-DTW library: argument validation, workspace
// layout and kernel sequencing.  Declarations and contracts: include/sdtw.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "sdtw.h"
#include "sdtw_kernels.h"

namespace {

using sdtw::DPArgs;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Private workspace layout.  Every region starts on a 256-byte boundary.
// The cell arrays use the band-step layout of sdtw_kernels.h.
struct Layout {
  int64_t nbands = 0, nseg = 0, S = 0;
  size_t ctrl = 0, ctrl_words = 0;  // ticket, done, per-segment progress
  size_t err_word = 0;              // index of the error word among the control words
  size_t loss64 = 0;                // fp64 [B]
  size_t H = 0;                     // fp64 [2, B, nseg, M] segment hand-off rows
  size_t R = 0;                     // fp64 band-step forward state
  size_t R2 = 0;                    // fp64 band-step reverse soft-min parts (unfused, concurrent)
  bool seq = false;                 // low-memory unfused: sweeps in turn, E formed by the reverse
  size_t eflag = 0;                 // index of the E-formed flag among the control words (seq)
  size_t part = 0;                  // fp32 split partial sums of the chain rule (unfused)
  size_t cnt_rows = 0, cnt_cols = 0;  // word offsets of the chain split counters
  size_t dist = 0;                  // fp32 band-step distances, then E (unfused)
  unsigned hcols = 0;               // inference: hand-off ring columns (0: whole rows)
  // Checkpointed training: groups of G bands, ng groups, ng-1 checkpoint
  // rows; control words of the group launches (2 + B*G, then the word
  // holding M and a sink word), checkpoint rows [B][ng-1][M + 2*kCkPad],
  // two reverse hand-off rows [2][B][M], and the X of one group (band-step).
  int64_t G = 0, ng = 0;
  size_t gctrl = 0, ckpt = 0, rh = 0;
  size_t total = 0;
};

// Bands per checkpoint group: about the square root of the band count, so
// the checkpoint rows (one per group) and the recomputed group of bands
// both stay near sqrt(N/64) rows of M states per pair.
int64_t ckpt_group(int64_t nbands) {
  int64_t g = 1;
  while (g * g < nbands) ++g;
  return g;
}

// Inference mode hands each band's bottom row to the next band either whole
// (B*nbands*M*8 bytes; tickets run band-major, the fastest order when the
// workgroups of all pairs do not fit on the GPU at once) or through rings of
// kHRing columns (B*nbands*kHRing*8 bytes; a band may then wait on the band
// below, so tickets run pair-major and every band of a pair must be resident
// together: at most one workgroup per CU of the 256).  Rings are taken when
// they cost no speed, i.e. all B*nbands workgroups fit at once, or when whole
// rows would exceed both kInferRowsFree and the size of the inputs.
constexpr int64_t kInferCUs = 256;
constexpr size_t kInferRowsFree = size_t(16) << 20;

unsigned infer_ring_cols(int64_t B, int64_t nbands, int64_t M, int64_t N, int64_t D) {
  if (M <= (int64_t)sdtw::kHRing || nbands > kInferCUs) return 0;
  const size_t rows = (size_t)B * (size_t)nbands * (size_t)M * 8;
  const size_t inputs = (size_t)B * (size_t)(N + M) * (size_t)D * 4;
  const bool all_resident = B * nbands <= kInferCUs;
  const bool rows_too_big = rows > kInferRowsFree && rows > inputs;
  return (all_resident || rows_too_big) ? sdtw::kHRing : 0;
}

bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

bool sizes_ok(int64_t B, int64_t N, int64_t M, int64_t D) {
  if (B < 1 || N < 1 || M < 1 || D < 1) return false;
  if (B > 65535) return false;                 // grid-dimension limit
  if (N > (int64_t(1) << 31) || M > (int64_t(1) << 31) || D > (int64_t(1) << 24))
    return false;
  size_t nm, bnm, bytes;
  if (!mul_ok((size_t)N, (size_t)M, &nm)) return false;
  if (!mul_ok(nm, (size_t)B, &bnm)) return false;
  if (!mul_ok(bnm, 64, &bytes)) return false;  // R + Dist + padding, generously
  return bytes < (SIZE_MAX >> 2);
}

bool make_layout(int64_t B, int64_t N, int64_t M, int64_t D, int mode, Layout* L) {
  if (!sizes_ok(B, N, M, D) ||
      (mode != SDTW_MODE_UNFUSED && mode != SDTW_MODE_FUSED && mode != SDTW_MODE_INFERENCE &&
       mode != SDTW_MODE_CHECKPOINT && mode != SDTW_MODE_UNFUSED_LOWMEM))
    return false;
  L->nbands = (N + 63) / 64;
  if (mode == SDTW_MODE_CHECKPOINT) {
    // The loss-only forward (plus checkpoint rows), then per group a forward
    // over the group's rows that keeps X and a reverse over them.
    if (sdtw::fused_bands_per_wg(D) == 0) return false;
    L->nseg = L->nbands;
    L->hcols = infer_ring_cols(B, L->nbands, M, N, D);
    L->S = sdtw::band_stride(M);
    L->G = ckpt_group(L->nbands);
    L->ng = (L->nbands + L->G - 1) / L->G;
    const size_t row = L->hcols ? L->hcols : (size_t)M;
    const size_t hrow = (size_t)L->nbands * row > (size_t)L->G * (size_t)M
                            ? (size_t)L->nbands * row : (size_t)L->G * (size_t)M;
    size_t off = 0;
    L->ctrl = off;
    L->gctrl = 2 + 2 * (size_t)B * (size_t)L->nseg;
    L->ctrl_words = L->gctrl + 2 + (size_t)B * (size_t)L->G + 2;
    L->err_word = L->ctrl_words++;
    off += align_up(L->ctrl_words * 4);
    L->loss64 = off;
    off += align_up((size_t)B * 8);
    L->H = off;
    off += align_up((size_t)B * hrow * 8);
    L->ckpt = off;
    off += align_up((size_t)B * (size_t)(L->ng - 1) * ((size_t)M + 2 * sdtw::kCkPad) * 8);
    L->rh = off;
    off += align_up(2 * (size_t)B * (size_t)M * 8);
    L->R = off;
    off += align_up((size_t)sdtw::band_array_elems(B * L->G, L->S, M) * 8);
    L->total = off;
    return true;
  }
  if (mode == SDTW_MODE_INFERENCE) {
    // Loss only: control words, the final states and the hand-off rows.
    if (sdtw::fused_bands_per_wg(D) == 0) return false;
    L->nseg = L->nbands;
    L->hcols = infer_ring_cols(B, L->nbands, M, N, D);
    const size_t row = L->hcols ? L->hcols : (size_t)M;
    size_t off = 0;
    L->ctrl = off;
    L->ctrl_words = 2 + 2 * (size_t)B * (size_t)L->nseg;
    L->err_word = L->ctrl_words++;
    off += align_up(L->ctrl_words * 4);
    L->loss64 = off;
    off += align_up((size_t)B * 8);
    L->H = off;
    off += align_up((size_t)B * (size_t)L->nseg * row * 8);
    L->total = off;
    return true;
  }
  const int bpw = mode == SDTW_MODE_FUSED ? sdtw::fused_bands_per_wg(D) : sdtw::kBandsPerWG;
  if (bpw == 0) return false;  // fused mode: D beyond what the kernels hold on chip
  L->nseg = (L->nbands + bpw - 1) / bpw;
  const bool unfused = mode == SDTW_MODE_UNFUSED || mode == SDTW_MODE_UNFUSED_LOWMEM;
  L->S = sdtw::band_stride(M);
  const size_t cells = (size_t)sdtw::band_array_elems(B * L->nbands, L->S, M);
  size_t off = 0;
  L->ctrl = off;
  // DP words (two halves of ticket, done, progress), then the counters of
  // the chain rule's split sums (one per band, one per 64-column block).
  L->cnt_rows = 2 * (2 + (size_t)B * (size_t)L->nseg);
  L->cnt_cols = L->cnt_rows + (size_t)B * (size_t)L->nbands;
  L->ctrl_words = L->cnt_cols + (size_t)B * (size_t)((M + 63) / 64);
  L->eflag = L->ctrl_words++;
  L->err_word = L->ctrl_words++;
  off += align_up(L->ctrl_words * 4);
  L->loss64 = off;
  off += align_up((size_t)B * 8);
  L->H = off;
  off += align_up(2 * (size_t)B * (size_t)L->nseg * (size_t)M * 8);
  L->R = off;
  off += align_up(cells * 8);
  if (unfused) {
    // Low-memory unfused: the sweeps one after the other, the reverse one
    // forming E over the distances, so T' is never stored.
    L->seq = mode == SDTW_MODE_UNFUSED_LOWMEM;
    if (!L->seq) {
      L->R2 = off;
      off += align_up(cells * 8);
    }
    L->part = off;
    off += align_up(sdtw::chain_part_floats(B, N, M, D) * 4);
    // Distances, then E or the row pass's dy shares.
    const size_t shares = sdtw::chain_share_floats(B, N, M, D);
    L->dist = off;
    off += align_up((cells > shares ? cells : shares) * 4);
  }
  L->total = off;
  return true;
}

bool gamma_ok(float g) { return isfinite(g) && g > 0.f; }

// Test hook of sdtw_debug_wait_limit: replaces the kernels' wait caps (0 =
// the built-in caps).
std::atomic<unsigned> g_wait_cap{0};

// Hand-off row entries of the unfused and fused training layouts.
int64_t hrow_doubles(const Layout& L, int64_t B, int64_t M) { return 2 * B * L.nseg * M; }

// Control words: the unfused launch (both sweeps) uses them from the start;
// the fused sweeps run as separate launches, the forward one on the first
// half and the reverse one on the second.  Every launch leaves its words
// zeroed when it finishes.
DPArgs dp_args(const Layout& L, char* ws, const float* x, const float* y,
               int64_t B, int64_t N, int64_t M, int64_t D, float gamma,
               bool reverse) {
  DPArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.y = y;
  a.ctrl = reinterpret_cast<unsigned*>(ws + L.ctrl) + (reverse ? 2 + B * L.nseg : 0);
  a.loss64 = reinterpret_cast<double*>(ws + L.loss64);
  a.H = reinterpret_cast<double*>(ws + L.H);
  a.R = L.R ? reinterpret_cast<double*>(ws + L.R) : nullptr;
  a.R2 = L.R2 ? reinterpret_cast<double*>(ws + L.R2) : nullptr;
  a.dsk = L.dist ? reinterpret_cast<float*>(ws + L.dist) : nullptr;
  a.N = N;
  a.S = L.S;
  a.M = M;
  a.D = D;
  a.B = (int)B;
  a.nbands = (int)L.nbands;
  a.nseg = (int)L.nseg;
  a.err = reinterpret_cast<unsigned*>(ws + L.ctrl) + L.err_word;
  a.wait_cap = g_wait_cap.load(std::memory_order_relaxed);
  a.sweeps = sdtw::kSweepsBoth;
  a.eflag = reinterpret_cast<unsigned*>(ws + L.ctrl) + L.eflag;
  const double g = (double)gamma;
  a.k2 = M_LOG2E / g;
  a.g_ln2 = g * M_LN2;
  return a;
}

// Checkpointed backward: the reverse sweep runs group by group from the
// bottom of the grid (reverse bands hG .. hG+G-1), each group after a
// forward sweep that recomputes X of the group's rows from the checkpoint
// row above them (the grid's top boundary for the last group).  The reverse
// sweep's row between groups passes through the two hand-off rows in turn.
int backward_checkpointed(const Layout& L, char* ws, const float* x, const float* y,
                          int64_t B, int64_t N, int64_t M, int64_t D, float gamma,
                          const float* grad_loss, float* grad_x, float* grad_y, float* align,
                          hipStream_t s) {
  unsigned* ctrl = reinterpret_cast<unsigned*>(ws + L.ctrl);
  unsigned* gctrl = ctrl + L.gctrl;
  unsigned* full = gctrl + 2 + (size_t)B * (size_t)L.G;
  double* ckpt = reinterpret_cast<double*>(ws + L.ckpt);
  double* rh = reinterpret_cast<double*>(ws + L.rh);
  const int64_t G = L.G, ng = L.ng, nb = L.nbands;
  hipError_t e = hipSuccess;
  if (grad_y) e = sdtw::launch_zero_f32(grad_y, B * M * D, s);
  // Group control words start cleared (each launch leaves them so); the
  // full word tells a range launch that its top row is complete.
  if (e == hipSuccess) e = sdtw::launch_zero_u32(gctrl, 2 + B * G, s);
  if (e == hipSuccess) e = sdtw::launch_fill_u32(full, 1, (unsigned)M, s);
  // The rows handed between the bands of a group launch carry their own
  // validity: whole rows come back from the forward set to kHEmpty; after a
  // forward through rings they are set here.  Every launch leaves them so.
  if (e == hipSuccess && L.hcols != 0)
    e = sdtw::launch_clear(nullptr, 0, reinterpret_cast<double*>(ws + L.H), B * G * M, s);
  DPArgs base = dp_args(L, ws, x, y, B, N, M, D, gamma, false);
  base.hvalid = 1;
  base.ctrl = gctrl;
  base.nbands = (int)G;                      // bands of the X buffer
  base.full_word = full;
  base.sink_word = full + 1;
  for (int64_t h = 0; h < ng && e == hipSuccess; ++h) {
    const int64_t r1 = N - 64 * h * G;       // original rows [r0, r1)
    const int64_t r0 = N - 64 * (h + 1) * G > 0 ? N - 64 * (h + 1) * G : 0;
    DPArgs f = base;
    f.row0 = f.xrow0 = r0;
    f.nseg = (int)((r1 - r0 + 63) / 64);
    f.top_row = h + 1 < ng ? ckpt + h * (M + 2 * sdtw::kCkPad) + sdtw::kCkPad : nullptr;
    f.top_ld = (ng - 1) * (M + 2 * sdtw::kCkPad);
    e = sdtw::launch_fused_range(f, false, s);
    if (e != hipSuccess) break;
    DPArgs r = base;
    r.row0 = 64 * h * G;
    r.xrow0 = r0;
    r.nseg = (int)(nb - h * G < G ? nb - h * G : G);
    r.top_row = h > 0 ? rh + ((h - 1) & 1) * B * M : nullptr;
    r.top_ld = M;
    r.bot_row = h + 1 < ng ? rh + (h & 1) * B * M : nullptr;
    r.gl = grad_loss;
    r.gx = grad_x;
    r.gy = grad_y;
    r.align = align;
    e = sdtw::launch_fused_range(r, true, s);
  }
  return e == hipSuccess ? SDTW_OK : SDTW_ERR_HIP;
}

int check_ws(const Layout& L, void* ws, size_t bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return SDTW_ERR_INVALID_ARG;
  if (bytes < L.total) return SDTW_ERR_WORKSPACE;
  return SDTW_OK;
}

}  // namespace

namespace sdtw {

// Body of sdtw_forward (also behind the allocation-free loss-only entry point).
int forward_impl(const float* x, const float* y, int64_t B, int64_t N, int64_t M, int64_t D,
                 float gamma, int mode, void* workspace, size_t workspace_bytes, float* loss,
                 void* stream) {
  if (!x || !y || !loss || !gamma_ok(gamma)) return SDTW_ERR_INVALID_ARG;
  Layout L;
  if (!make_layout(B, N, M, D, mode, &L)) return SDTW_ERR_INVALID_ARG;
  int st = check_ws(L, workspace, workspace_bytes);
  if (st != SDTW_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  DPArgs a = dp_args(L, ws, x, y, B, N, M, D, gamma, false);
  a.loss = loss;
  const bool fused = mode == SDTW_MODE_FUSED;
  unsigned* ctrl = reinterpret_cast<unsigned*>(ws + L.ctrl);
  // A fresh workspace holds garbage: the control words are cleared once per
  // forward (later launches find them cleared by the kernels), by the
  // distance kernel where there is one.
  hipError_t e = hipSuccess;
  if (mode == SDTW_MODE_INFERENCE || mode == SDTW_MODE_CHECKPOINT) {
    if (L.hcols) {
      // Ring hand-off needs every band of a pair resident at once (one
      // workgroup per band, at least one workgroup per CU).
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return SDTW_ERR_HIP;
      if ((int64_t)cus < L.nseg) return SDTW_ERR_UNSUPPORTED;
    }
    if (L.hcols == 0) {
      // Whole hand-off rows carry their own validity (set to kHEmpty here;
      // the checkpointed backward's launches use counts and overwrite them).
      e = sdtw::launch_clear(ctrl, (int64_t)L.ctrl_words, a.H, B * L.nseg * M, s);
      a.hvalid = 1;
    } else {
      e = sdtw::launch_zero_u32(ctrl, (int64_t)L.ctrl_words, s);
    }
    if (mode == SDTW_MODE_CHECKPOINT) {
      a.R = nullptr;
      a.ckpt = reinterpret_cast<double*>(ws + L.ckpt);
      a.ck_span = 64 * L.G;
      a.nck = (int)(L.ng - 1);
    }
    if (e == hipSuccess) e = sdtw::launch_infer(a, L.hcols, s);
  } else if (fused) {
    // The hand-off rows start as kHEmpty; every sweep leaves them so, which
    // the backward's sweep relies on.
    e = sdtw::launch_clear(ctrl, (int64_t)L.ctrl_words, a.H, hrow_doubles(L, B, M), s);
    a.hvalid = 1;
    if (e == hipSuccess) e = sdtw::launch_dp_fused(a, false, s);
  } else {
    // Unfused: both sweeps at once; the loss comes from the forward one, and
    // the reverse one leaves what the backward needs besides the forward
    // state.  Low-memory unfused: the forward sweep alone (the backward runs
    // the reverse).  The distance kernel also clears the control words,
    // E-formed flag included.
    e = sdtw::launch_dist_skew(x, y, a.dsk, B, N, M, D, L.S, ctrl, (int64_t)L.ctrl_words, a.H,
                               hrow_doubles(L, B, M), s);
    a.hvalid = 1;
    a.sweeps = L.seq ? sdtw::kSweepForward : sdtw::kSweepsBoth;
    if (e == hipSuccess) e = sdtw::launch_dp_both(a, s);
  }
  return e == hipSuccess ? SDTW_OK : SDTW_ERR_HIP;
}

}  // namespace sdtw

extern "C" {

int sdtw_abi_version(void) { return SDTW_ABI_VERSION; }

const char* sdtw_status_string(int status) {
  switch (status) {
    case SDTW_OK: return "ok";
    case SDTW_ERR_INVALID_ARG: return "invalid argument";
    case SDTW_ERR_WORKSPACE: return "workspace too small";
    case SDTW_ERR_HIP: return "HIP runtime error";
    case SDTW_ERR_UNSUPPORTED: return "unsupported request";
    case SDTW_ERR_STALLED: return "a hand-off wait inside a kernel gave up; outputs set to NaN";
    default: return "unknown status";
  }
}

size_t sdtw_workspace_bytes(int64_t B, int64_t N, int64_t M, int64_t D, int mode) {
  Layout L;
  if (!make_layout(B, N, M, D, mode, &L)) return 0;
  return L.total;
}

int sdtw_dist(const float* x, const float* y, float* dist, int64_t B, int64_t N,
              int64_t M, int64_t D, void* stream) {
  if (!x || !y || !dist || !sizes_ok(B, N, M, D)) return SDTW_ERR_INVALID_ARG;
  hipError_t e = sdtw::launch_dist(x, y, dist, B, N, M, D, (hipStream_t)stream);
  return e == hipSuccess ? SDTW_OK : SDTW_ERR_HIP;
}

int sdtw_forward(const float* x, const float* y, int64_t B, int64_t N, int64_t M,
                 int64_t D, float gamma, int mode, void* workspace,
                 size_t workspace_bytes, float* loss, void* stream) {
  return sdtw::forward_impl(x, y, B, N, M, D, gamma, mode, workspace, workspace_bytes, loss,
                            stream);
}

int sdtw_backward(const float* x, const float* y, int64_t B, int64_t N, int64_t M,
                  int64_t D, float gamma, int mode, void* workspace,
                  size_t workspace_bytes, const float* grad_loss, float* grad_x,
                  float* grad_y, float* align, void* stream) {
  if (!x || !y || !grad_loss || !gamma_ok(gamma)) return SDTW_ERR_INVALID_ARG;
  Layout L;
  if (!make_layout(B, N, M, D, mode, &L)) return SDTW_ERR_INVALID_ARG;
  int st = check_ws(L, workspace, workspace_bytes);
  if (st != SDTW_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  if (mode == SDTW_MODE_INFERENCE) return SDTW_ERR_UNSUPPORTED;  // nothing kept to go back on
  if (mode == SDTW_MODE_CHECKPOINT) {
    if (!grad_x && !grad_y && !align) return SDTW_OK;
    return backward_checkpointed(L, ws, x, y, B, N, M, D, gamma, grad_loss, grad_x, grad_y,
                                 align, (hipStream_t)stream);
  }
  DPArgs a = dp_args(L, ws, x, y, B, N, M, D, gamma, mode == SDTW_MODE_FUSED);
  if (mode == SDTW_MODE_FUSED) {
    // One reverse sweep per slice of D; it writes dx, adds into dy and, if
    // asked, writes E.  Nothing to compute when no output is requested.
    if (!grad_x && !grad_y && !align) return SDTW_OK;
    a.gl = grad_loss;
    a.gx = grad_x;
    a.gy = grad_y;
    a.align = align;
    hipError_t e = hipSuccess;
    a.hvalid = 1;   // the forward left the hand-off rows at kHEmpty
    if (grad_y) e = sdtw::launch_zero_f32(grad_y, B * M * D, s);
    if (e == hipSuccess) e = sdtw::launch_dp_fused(a, true, s);
    return e == hipSuccess ? SDTW_OK : SDTW_ERR_HIP;
  }
  // Unfused: both sweeps ran in the forward; the chain rule forms E from
  // their states (the distances are not read again).  Low-memory unfused:
  // the reverse sweep forms E over the distances, once per forward (a
  // repeated backward finds the E-formed flag set and reuses E); the chain
  // rule reads it.  Either way repeated backward calls on one forward are
  // all valid.
  if (!grad_x && !grad_y && !align) return SDTW_OK;
  unsigned* ctrl = reinterpret_cast<unsigned*>(ws + L.ctrl);
  hipError_t e = hipSuccess;
  if (L.seq) {
    a.sweeps = sdtw::kSweepReverseE;
    a.hvalid = 1;   // the reverse half of the hand-off rows is still at kHEmpty
    e = sdtw::launch_dp_both(a, s);
  }
  if (e == hipSuccess)
    e = sdtw::launch_chain(a.dsk, a.R, a.R2, a.loss64, x, y, grad_loss, grad_x, grad_y, B, N,
                           M, D, L.S, reinterpret_cast<float*>(ws + L.part), ctrl + L.cnt_rows,
                           ctrl + L.cnt_cols, align != nullptr, L.seq, s);
  if (e == hipSuccess && align) e = sdtw::launch_unskew(a.dsk, align, B, N, M, L.S, s);
  return e == hipSuccess ? SDTW_OK : SDTW_ERR_HIP;
}

int sdtw_workspace_status(const void* workspace, size_t workspace_bytes, int64_t B,
                          int64_t N, int64_t M, int64_t D, int mode, void* stream) {
  Layout L;
  if (!make_layout(B, N, M, D, mode, &L)) return SDTW_ERR_INVALID_ARG;
  int st = check_ws(L, const_cast<void*>(workspace), workspace_bytes);
  if (st != SDTW_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  unsigned word = 0;
  const char* src = static_cast<const char*>(workspace) + L.ctrl + 4 * L.err_word;
  if (hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return SDTW_ERR_HIP;
  return word ? SDTW_ERR_STALLED : SDTW_OK;
}

int sdtw_debug_wait_limit(int64_t polls) {
  if (polls < 0 || polls > (int64_t)0xffffffffLL) return SDTW_ERR_INVALID_ARG;
  g_wait_cap.store((unsigned)polls, std::memory_order_relaxed);
  return SDTW_OK;
}

}  // extern "C"

/*
 * sdtw.h -- C ABI of the MI355X (gfx950) Soft-DTW library (libsdtw.so).
 *
 * Operation.  Soft-DTW (Cuturi & Blondel, ICML 2017; credited in the
 * "Acknowledgments" of the README "SoftDTW-CUDA (PyTorch + Numba)") between
 * x[b] (N x D) and y[b] (M x D) for every pair b of a batch:
 *
 *   Dist[b,i,j] = ||x[b,i,:] - y[b,j,:]||^2            (squared Euclidean)
 *   R[0,0] = 0,  R[i,0] = R[0,j] = +inf,
 *   R[i,j] = Dist[b,i-1,j-1] + softmin_g(R[i-1,j-1], R[i-1,j], R[i,j-1]),
 *   softmin_g(a) = -g log sum_k exp(-a_k/g),        loss[b] = R[N,M].
 *
 * The gradient is the alignment matrix E = dloss/dDist, obtained by a
 * log-space backward recursion with the exponential taken at the end (review
 * page "SoftDTW-CUDA-Torch: Memory-Efficient GPU-Accelerated Soft Dynamic Time
 * Warping for PyTorch", section "Proposed method"), pushed through Dist:
 *   dx[b,i] = 2 gl[b] sum_j E[i,j] (x_i - y_j),
 *   dy[b,j] = 2 gl[b] sum_i E[i,j] (y_j - x_i).
 *
 * Modes (README "Usage": unfused = explicit distance tensor; "Fused Mode" = no
 * distance tensor; "Limitations": fused supports squared Euclidean only):
 *   SDTW_MODE_UNFUSED  materialises Dist (fp32, B x N x M) in the workspace;
 *                      the forward runs the forward and the reverse sweep of
 *                      the dynamic programme at once and keeps both states
 *                      (fp64); the backward forms E from them and applies
 *                      the chain rule, using the distance region for E (or,
 *                      for D <= 64 without an alignment output, for each
 *                      64-row band's share of grad_y).  About 20 bytes of
 *                      workspace per cell: 8 + 8 + 4 bytes for each of M + 63
 *                      columns (rounded up to 16) of every row.
 *   SDTW_MODE_UNFUSED_LOWMEM the unfused computation with the sweeps one
 *                      after the other: the forward runs the forward sweep
 *                      and keeps its state; the backward runs the reverse
 *                      sweep, which forms E over the distances (once per
 *                      forward: a repeated backward reuses it), then the
 *                      chain rule with the column pass for grad_y.  About
 *                      12 bytes per cell; slower than SDTW_MODE_UNFUSED
 *                      (one sweep at a time keeps fewer loads in flight),
 *                      faster than SDTW_MODE_FUSED.  Loss, E and grad_x are
 *                      bitwise those of SDTW_MODE_UNFUSED, grad_y too where
 *                      that mode takes the column pass (D > 64 or align).
 *   SDTW_MODE_FUSED    recomputes distances from x and y inside the dynamic
 *                      programme; no B x N x M distance or E tensor exists.
 *                      Supports D <= 256 (sdtw_workspace_bytes returns 0 and
 *                      the calls return SDTW_ERR_INVALID_ARG beyond that).
 *   SDTW_MODE_INFERENCE the loss alone (the README's "When to Use Each Mode"
 *                      names inference as a use): distances recomputed as
 *                      in fused mode and no DP state kept.  The workspace
 *                      holds control words and the rows handed between
 *                      64-row bands: whole rows (B*ceil(N/64)*M*8 bytes)
 *                      while that is at most 16 MiB or the inputs' size,
 *                      else rings of 512 columns (B*ceil(N/64)*512*8 bytes,
 *                      O(B*N)); rings are also used whenever all the pairs'
 *                      bands fit on 256 CUs at once.  Rings need N <= 16384.
 *                      D <= 256.  sdtw_backward returns SDTW_ERR_UNSUPPORTED
 *                      for it, and with rings sdtw_forward returns
 *                      SDTW_ERR_UNSUPPORTED on a GPU with fewer CUs than
 *                      the pair has bands (they must all be resident).  The
 *                      loss is bitwise the one the other modes return.
 *   SDTW_MODE_CHECKPOINT training without the B x N x M forward state
 *                      (distances recomputed as in fused mode, D <= 256):
 *                      the forward is the inference one and also keeps one
 *                      checkpoint row (fp64, M states) every G = ceil(sqrt(
 *                      ceil(N/64))) bands; the backward runs the reverse
 *                      sweep group by group of G bands from the bottom,
 *                      each after a forward sweep that recomputes the
 *                      group's states from the checkpoint row above it.
 *                      Workspace about B*(G*64*(M+78)*8 + N/(64G)*M*8)
 *                      bytes, plus the inference mode's hand-off rows (the
 *                      same CU condition applies to its forward).  Loss, alignment matrix and grad_x are
 *                      bitwise those of SDTW_MODE_FUSED (same arithmetic on
 *                      the same values); the backward is repeatable.
 * The unfused and fused modes keep the forward DP state (fp64, B x N x M)
 * for the backward.
 * Distances are accumulated in fp64 and rounded once to fp32 in both modes,
 * so fused and unfused see identical distances, losses and alignment
 * matrices (gradients agree to rounding: they are summed in other orders).
 *
 * Conventions for every entry point:
 *  - x is [B,N,D], y is [B,M,D], fp32, row-major and contiguous, in device
 *    memory; every other array argument is a device pointer too.
 *  - B, N, M, D >= 1 (the README's "empty sequences" are rejected); lengths
 *    are unbounded apart from memory; products such as B*N*M must fit int64.
 *  - gamma must be finite and > 0.
 *  - All work is enqueued on `stream` (a hipStream_t; 0 = the null stream)
 *    without host synchronisation.  Arguments are validated on the host before
 *    any HIP call; invalid calls return an error and enqueue nothing.  Faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - Hand-offs between workgroups and waves are bounded waits: a wave that
 *    polls a counter or a hand-off row far longer than any normal run needs
 *    (about 0.1 s on chip, seconds on a global row) gives up so that every
 *    kernel still exits.  Such a call cannot have correct results: the
 *    launch sets its outputs (loss, grad_x, grad_y, align, and the kept
 *    final state, so a later backward is NaN too) to NaN, and
 *    sdtw_workspace_status reports SDTW_ERR_STALLED until the next forward
 *    on the workspace.  The ring hand-off of the inference and checkpointed
 *    forwards (see the modes) needs every band of a pair resident at once:
 *    kernels of other streams holding the CUs for longer than the cap make
 *    it stall this way instead of hanging.
 *  - The library never allocates device memory; the caller owns every buffer
 *    passed in.  Process-wide state is limited to: the launch-timing record
 *    list (sdtw_timing, off by default, guarded by a mutex), the
 *    per-device scratch array of sdtw_forward_static with its resolved
 *    addresses, and the wait limit of sdtw_debug_wait_limit.  Calls on
 *    distinct workspaces may run concurrently on distinct streams.  Nothing
 *    is printed.
 */
#ifndef SDTW_H
#define SDTW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDTW_ABI_VERSION 3

typedef enum {
    SDTW_OK = 0,
    SDTW_ERR_INVALID_ARG = 1, /* bad size, gamma, pointer or mode          */
    SDTW_ERR_WORKSPACE = 2,   /* workspace_bytes below sdtw_workspace_bytes */
    SDTW_ERR_HIP = 3,         /* a HIP runtime call or launch failed        */
    SDTW_ERR_UNSUPPORTED = 4, /* request outside what the library supports  */
    SDTW_ERR_STALLED = 5      /* a hand-off wait inside a kernel gave up    */
} sdtw_status_t;

typedef enum {
    SDTW_MODE_UNFUSED = 0,
    SDTW_MODE_FUSED = 1,
    SDTW_MODE_INFERENCE = 2,
    SDTW_MODE_CHECKPOINT = 3,
    SDTW_MODE_UNFUSED_LOWMEM = 4
} sdtw_mode_t;

/* Version of this ABI (SDTW_ABI_VERSION). */
int sdtw_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *sdtw_status_string(int status);

/* Bytes of device workspace that sdtw_forward / sdtw_backward need for this
 * problem and mode (a multiple of 256; the pointer must be 256-byte aligned).
 * Returns 0 for invalid sizes or mode.  Layout is private to the library. */
size_t sdtw_workspace_bytes(int64_t B, int64_t N, int64_t M, int64_t D,
                            int mode);

/* Squared Euclidean distances dist[b,i,j] = ||x[b,i]-y[b,j]||^2 (fp32,
 * [B,N,M] row-major, caller-allocated), accumulated in fp64 and rounded once
 * (README "Usage", unfused mode's explicit distance computation; "Notes":
 * never negative). */
int sdtw_dist(const float *x, const float *y, float *dist, int64_t B,
              int64_t N, int64_t M, int64_t D, void *stream);

/* Forward pass: loss[b] = Soft-DTW(x[b], y[b]) (fp32, [B]).  Leaves in the
 * workspace what sdtw_backward needs (README "Usage": loss_fn(x, y) returns a
 * per-pair loss).  Soft-DTW can be negative (README "Notes").  The workspace
 * needs no clearing beforehand: the forward itself sets the control words and
 * hand-off rows its kernels and the backward's rely on. */
int sdtw_forward(const float *x, const float *y, int64_t B, int64_t N,
                 int64_t M, int64_t D, float gamma, int mode, void *workspace,
                 size_t workspace_bytes, float *loss, void *stream);

/* Backward pass for upstream gradients grad_loss[b] (fp32, [B]); the
 * workspace must be as sdtw_forward left it for the same arguments.
 * grad_x ([B,N,D]) and grad_y ([B,M,D]) are written (not accumulated); either
 * may be NULL to skip it.  align ([B,N,M] fp32), if not NULL, receives E
 * (every training mode; in the fused and checkpointed modes it is the only
 * B x N x M array written).  The backward never reads the distances again
 * (unfused mode overwrites them, with E formed from the two sweeps' states
 * or with the bands' shares of grad_y), so it may be repeated on one forward
 * in every training mode; with every output NULL it does nothing.  In the
 * fused and checkpointed modes grad_y is accumulated with atomic adds across
 * row bands, so its last bits may differ from run to run.  Inference mode:
 * SDTW_ERR_UNSUPPORTED. */
int sdtw_backward(const float *x, const float *y, int64_t B, int64_t N,
                  int64_t M, int64_t D, float gamma, int mode, void *workspace,
                  size_t workspace_bytes, const float *grad_loss,
                  float *grad_x, float *grad_y, float *align, void *stream);

/* Waits for `stream`, then reports whether a hand-off wait of the last
 * sdtw_forward / sdtw_backward on this workspace (same sizes and mode) gave
 * up: SDTW_OK, SDTW_ERR_STALLED (the outputs of that call were set to NaN),
 * SDTW_ERR_INVALID_ARG / SDTW_ERR_WORKSPACE as for sdtw_forward, or
 * SDTW_ERR_HIP if the copy of the workspace's error word failed.  The word
 * is cleared by every forward and kept by backwards. */
int sdtw_workspace_status(const void *workspace, size_t workspace_bytes,
                          int64_t B, int64_t N, int64_t M, int64_t D,
                          int mode, void *stream);

/* Test hook: a nonzero `polls` replaces the kernels' wait caps (polls of a
 * counter or of a hand-off row) for later calls from any thread; 0 restores
 * the built-in caps.  A tiny limit makes waits give up deliberately (every
 * kernel still exits; see SDTW_ERR_STALLED).  SDTW_ERR_INVALID_ARG for a
 * negative value or one above 2^32-1. */
int sdtw_debug_wait_limit(int64_t polls);

/* Size of the device array behind sdtw_forward_static (per GPU). */
#define SDTW_STATIC_SCRATCH_BYTES (16u << 20)

/* Loss-only forward (the same computation and result, bitwise, as
 * sdtw_forward in SDTW_MODE_INFERENCE) that allocates nothing and takes no
 * workspace: its workspace is a file-scope device array of
 * SDTW_STATIC_SCRATCH_BYTES per GPU, which the library's code object holds
 * on every GPU it runs on until the process ends.  For callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  x, y, loss and stream as for
 * sdtw_forward.  Returns SDTW_ERR_WORKSPACE when the inference workspace of
 * this problem (sdtw_workspace_bytes(..., SDTW_MODE_INFERENCE)) exceeds
 * SDTW_STATIC_SCRATCH_BYTES, and the other statuses as sdtw_forward.  Every
 * call on one GPU uses that GPU's single array: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by
 * the caller.  Calls that follow one another on a stream are safe: each
 * clears the control words it needs with kernels of its own (no memset
 * node).  Launches of this call are never timed (sdtw_timing). */
int sdtw_forward_static(const float *x, const float *y, int64_t B, int64_t N,
                        int64_t M, int64_t D, float gamma, float *loss,
                        void *stream);

/* Launch timing, off by default.  sdtw_timing(1) makes every kernel that
 * later sdtw_* calls (from any host thread of the process) enqueue be
 * bracketed by a pair of HIP events recorded on that call's stream;
 * sdtw_timing(0) stops recording.  Returns SDTW_OK.  Recording costs two
 * event creations per launch, so it is meant for measurement runs, not for
 * production loops. */
int sdtw_timing(int on);

/* Waits for the launches recorded since the previous collect (launches still
 * being enqueued by another thread are left for the next collect), writes
 * the names (static strings) and durations in milliseconds of the first
 * `cap` of them, in launch order, into names[] and ms[] (both
 * may be NULL when cap is 0), releases the events and returns how many
 * launches were recorded; -SDTW_ERR_HIP if an event could not be read (its
 * duration is then reported as -1). */
int sdtw_timing_collect(const char **names, float *ms, int cap);

#ifdef __cplusplus
}
#endif

#endif /* SDTW_H */
